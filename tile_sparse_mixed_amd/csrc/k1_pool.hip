// K1: block pooling and per-block E4M3 quantisation, one streaming pass over
// Q, K and V (HBM-bound).
//
// Per (b, h, key block J) one workgroup reads K_J and V_J once and writes
//   kbar_J, vbar_J   float32 block means (float64 sums / n_J; "Triage": a skipped
//                    tile is replaced by its block means),
//   kbar16, kbarlo   the K means as a bf16 pair hi + lo (hi = bf16(kbar), lo =
//                    bf16(kbar - hi)), the score operand of skipped tiles,
//   vbarT            the V means rounded to fp16, stored transposed per chunk of 64
//                    key blocks in vt_pos order (value operand of skipped tiles);
//                    the last block also zeroes the chunk's columns past Nk,
//   sk_J, sv_J       amax/448 (1 for an all-zero block),
//   k8               E4M3 codes of K_J, row-major with k8_pos d order,
//   vt               V_J as fp16, transposed ([d][key]) in the key order the
//                    fused kernel's P.V uses (vt_pos for 64-key blocks, vt16_pos
//                    for 16-key blocks, which the kernel gathers four at a time,
//                    natural order for 8-key blocks, gathered eight at a time),
//   vlow             the low tier's V operand, fl16(fl32(decode(E4M3(v * inv)) * sv)),
//                    in the same transposed layout.
// Per (b, h, query block I) one workgroup writes qbar_I, sq_I and iq_I = 448/amax.
// With the SKIM tier a third kernel writes MXFP4 copies of K and V (k1_mx4).
// For the price router both also write second moments from float64 sums of
// squares ("Triage": the router works from block statistics): per dimension
// the query mean square and the key variance, per block the key and value
// mean-square totals, the value variance total and the norm of the value mean.
#include "tattn_device.hpp"
#include "tattn_internal.hpp"

namespace tattn {
namespace {

constexpr int kThreads = 256;

// fl32(448 / a) and fl32(a / 448), correctly rounded: a float64 quotient of
// two floats rounded once to float equals the correctly rounded float quotient.
// An all-zero block gets 1 for both.
__device__ inline float inv448(float a) { return a == 0.0f ? 1.0f : static_cast<float>(448.0 / static_cast<double>(a)); }
__device__ inline float scale448(float a) { return a == 0.0f ? 1.0f : static_cast<float>(static_cast<double>(a) / 448.0); }

// Block-wide float max; `red` holds kThreads/64 floats.
__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; i++) r = __builtin_fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// Column sums of a block of `rows` real rows (<= BLK) of a [N, D] bf16 tensor
// slice starting at `base` (row stride sn elements).  Each thread keeps its
// ROWS_PER_THREAD row chunks of 8 values in `vals` (float) for later use.
// Returns, for threads t < D, the float64 column sum of column t.
template <int D, int BLK>
struct BlockLoad {
  static constexpr int CH = D / 8;              // 16-byte chunks per row
  static constexpr int RT = kThreads / CH;      // threads per column chunk
  static constexpr int RPT = (BLK + RT - 1) / RT;
  float vals[RPT][8];
};

template <int D, int BLK, bool MOM = false>
__device__ void load_block(const uint16_t* __restrict__ base, int64_t sn, int rows, BlockLoad<D, BLK>& bl,
                           double* __restrict__ red /* [RT][D] */, double& colsum, float& amax,
                           double* colsq = nullptr) {
  using BL = BlockLoad<D, BLK>;
  const int t = threadIdx.x;
  const int c = t % BL::CH, r0 = t / BL::CH;
  double acc[8], acc2[8];
#pragma unroll
  for (int e = 0; e < 8; e++) acc[e] = acc2[e] = 0.0;
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < BL::RPT; i++) {
    const int r = r0 + i * BL::RT;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (r < rows && r < BLK) raw = *reinterpret_cast<const uint4*>(base + (int64_t)r * sn + c * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float f = __uint_as_float(e & 1 ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
      bl.vals[i][e] = f;
      acc[e] += static_cast<double>(f);
      if (MOM) acc2[e] += static_cast<double>(f) * static_cast<double>(f);   // exact product of bf16 values
      mx = __builtin_fmaxf(mx, __builtin_fabsf(f));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; e++) red[r0 * D + c * 8 + e] = acc[e];
  amax = mx;
  __syncthreads();
  colsum = 0.0;
  if (t < D) {
    double s = 0.0;
    for (int i = 0; i < BL::RT; i++) s += red[i * D + t];
    colsum = s;
  }
  __syncthreads();
  if (MOM) {   // the same reduction for the column sums of squares
#pragma unroll
    for (int e = 0; e < 8; e++) red[r0 * D + c * 8 + e] = acc2[e];
    __syncthreads();
    *colsq = 0.0;
    if (t < D) {
      double s = 0.0;
      for (int i = 0; i < BL::RT; i++) s += red[i * D + t];
      *colsq = s;
    }
    __syncthreads();
  }
}

// Block-wide float64 sum; `red` holds kThreads/64 doubles.
__device__ double block_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; i++) r += red[i];
  __syncthreads();
  return r;
}

// Second moments of a block column from its float64 sums (threads t < D):
// mean square S2/n and variance max(S2/n - (S1/n)^2, 0), each rounded once per
// operation (no fused multiply-add), as the price router's statistics define.
struct ColMoments {
  double mean, msq, var;
};
__device__ inline ColMoments col_moments(double s1, double s2, int n) {
  const double dn = static_cast<double>(n);
  ColMoments m;
  m.mean = s1 / dn;
  m.msq = s2 / dn;
  m.var = fmax(__dsub_rn(m.msq, __dmul_rn(m.mean, m.mean)), 0.0);
  return m;
}

template <int D, int BK, bool MOM>
__global__ __launch_bounds__(kThreads) void k1_kv(PoolArgs a) {
  static_assert(BK == 64 || BK == 16 || BK == 8, "key blocks are 64, 16 or 8 keys");
  constexpr int QR = BK / 8;   // 16-byte chunks per stored row of BK keys
  using BL = BlockLoad<D, BK>;
  __shared__ double red[BL::RT * D];
  __shared__ float fred[kThreads / 64];
  __shared__ double dred[kThreads / 64];
  __shared__ uint16_t tileT[BK * D];   // V block as bf16, [key][d], for the transposed stores

  const Dims& dm = a.d;
  const int bh = blockIdx.x / dm.Nk, J = blockIdx.x % dm.Nk;
  const int b = bh / dm.H, h = bh % dm.H;
  const int rows = min(BK, dm.N - J * BK);
  const int64_t off = (int64_t)b * dm.sb + (int64_t)h * dm.sh + (int64_t)J * BK * dm.sn;
  unsigned char* ws = a.ws;
  float* kbar = reinterpret_cast<float*>(ws + a.L.kbar) + ((int64_t)bh * dm.Nk + J) * D;
  float* vbar = reinterpret_cast<float*>(ws + a.L.vbar) + ((int64_t)bh * dm.Nk + J) * D;
  unsigned char* slab = ws + a.L.slab + (int64_t)bh * a.L.sl.bytes;
  uint16_t* kbar16 = reinterpret_cast<uint16_t*>(slab + a.L.sl.kbhi) + (int64_t)J * D;
  uint16_t* kbarlo = reinterpret_cast<uint16_t*>(slab + a.L.sl.kblo) + (int64_t)J * D;
  uint16_t* vbarT = reinterpret_cast<uint16_t*>(slab + a.L.sl.vbarT) + (int64_t)(J / 64) * 64 * D;
  float* sk = reinterpret_cast<float*>(ws + a.L.sk) + (int64_t)bh * dm.Nk + J;
  float* sv = reinterpret_cast<float*>(ws + a.L.sv) + (int64_t)bh * dm.Nk + J;
  unsigned char* k8 = slab + a.L.sl.k8 + (int64_t)J * BK * D;
  uint16_t* vlow = reinterpret_cast<uint16_t*>(slab + a.L.sl.vlow) + (int64_t)J * BK * D;
  uint16_t* vt = reinterpret_cast<uint16_t*>(slab + a.L.sl.vt) + (int64_t)J * BK * D;

  const int t = threadIdx.x;
  const int c = t % BL::CH, r0 = t / BL::CH;
  BL bl;
  double colsum, colsq = 0.0;
  float amax;
  const int64_t kb = (int64_t)bh * dm.Nk + J;   // this block's index in the [BH][Nk] statistics

  // ---- K: means, scale, codes (row-major, k8_pos order inside each row)
  load_block<D, BK, MOM>(a.k + off, dm.sn, rows, bl, red, colsum, amax, &colsq);
  if (t < D) {
    const float m = static_cast<float>(colsum / static_cast<double>(rows));
    kbar[t] = m;
    const uint16_t hi = f32_to_bf16(m);
    kbar16[t] = hi;
    kbarlo[t] = f32_to_bf16(m - bf16_to_f32(hi));   // the difference is exact in fp32
  }
  if (MOM) {   // key variance per dimension and the mean-square total
    const ColMoments cm = col_moments(colsum, colsq, rows);
    if (t < D) reinterpret_cast<float*>(a.ws + a.L.kvar)[kb * D + t] = static_cast<float>(cm.var);
    const double tot = block_sum_d(t < D ? cm.msq : 0.0, dred);
    if (t == 0) reinterpret_cast<float*>(a.ws + a.L.m2k)[kb] = static_cast<float>(tot);
  }
  amax = block_max(amax, fred);
  {
    const float inv = inv448(amax);
    if (t == 0) *sk = scale448(amax);
#pragma unroll
    for (int i = 0; i < BL::RPT; i++) {
      const int r = r0 + i * BL::RT;
      if (r >= BK) break;
      int w0 = 0, w1 = 0;
      w0 = cvt_fp8x2<false>(bl.vals[i][0] * inv, bl.vals[i][1] * inv, w0);
      w0 = cvt_fp8x2<true>(bl.vals[i][2] * inv, bl.vals[i][3] * inv, w0);
      w1 = cvt_fp8x2<false>(bl.vals[i][4] * inv, bl.vals[i][5] * inv, w1);
      w1 = cvt_fp8x2<true>(bl.vals[i][6] * inv, bl.vals[i][7] * inv, w1);
      // 8 consecutive d of one chunk land contiguously at k8_pos(8c)
      *reinterpret_cast<uint2*>(k8 + r * D + k8_pos(c * 8)) = make_uint2(w0, w1);
    }
  }

  // ---- V: means, scale, transposed codes and transposed bf16 values
  load_block<D, BK, MOM>(a.v + off, dm.sn, rows, bl, red, colsum, amax, &colsq);
  if (t < D) {
    const float m = static_cast<float>(colsum / static_cast<double>(rows));
    vbar[t] = m;
    vbarT[t * 64 + vt_pos(J & 63)] = f32_to_f16(m);
    if (J == dm.Nk - 1)   // finite zeros in the chunk's unused columns (they meet P = 0)
      for (int j = (J & 63) + 1; j < 64; j++) vbarT[t * 64 + vt_pos(j)] = 0;
  }
  if (MOM) {   // value variance total, mean-square total and the norm of the mean
    const ColMoments cm = col_moments(colsum, colsq, rows);
    const double tv = block_sum_d(t < D ? cm.var : 0.0, dred);
    const double tm = block_sum_d(t < D ? cm.msq : 0.0, dred);
    const double tn = block_sum_d(t < D ? __dmul_rn(cm.mean, cm.mean) : 0.0, dred);
    if (t == 0) {
      reinterpret_cast<float*>(a.ws + a.L.vvar)[kb] = static_cast<float>(tv);
      reinterpret_cast<float*>(a.ws + a.L.m2v)[kb] = static_cast<float>(tm);
      reinterpret_cast<float*>(a.ws + a.L.vnorm)[kb] = static_cast<float>(sqrt(tn));
    }
  }
#pragma unroll
  for (int i = 0; i < BL::RPT; i++) {
    const int r = r0 + i * BL::RT;
    if (r >= BK) break;
#pragma unroll
    for (int e = 0; e < 8; e++) tileT[r * D + c * 8 + e] = f32_to_bf16(bl.vals[i][e]);  // exact: inputs are bf16
  }
  amax = block_max(amax, fred);   // contains the barrier that publishes tileT
  const float inv = inv448(amax);
  if (t == 0) *sv = scale448(amax);
  // vt (fp16): D rows of BK keys = QR chunks of 8 elements; element e of row d
  // holds key vt_key<BK>(e).
  for (int u = t; u < D * QR; u += kThreads) {
    const int d = u / QR, q = u % QR;
    uint32_t w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; e2++) {
      uint32_t lohi[2];
#pragma unroll
      for (int z = 0; z < 2; z++) {
        const int key = vt_key<BK>(q * 8 + e2 * 2 + z);
        // bf16 -> fp16 is exact for |v| in [2^-14, 65504]; smaller values round
        lohi[z] = f32_to_f16(bf16_to_f32(tileT[key * D + d]));
      }
      w[e2] = lohi[0] | (lohi[1] << 16);
    }
    *reinterpret_cast<uint4*>(vt + d * BK + q * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // vlow: same layout as vt; element = fl16(fl32(decode(code)) * sv) of the E4M3 code
  // of v * inv (the hardware converter decodes exactly).
  const float svf = scale448(amax);
  for (int u = t; u < D * QR; u += kThreads) {
    const int d = u / QR, q = u % QR;
    uint32_t w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; e2++) {
      float f[2];
#pragma unroll
      for (int z = 0; z < 2; z++) {
        const int key = vt_key<BK>(q * 8 + e2 * 2 + z);
        f[z] = bf16_to_f32(tileT[key * D + d]) * inv;
      }
      const int code2 = cvt_fp8x2<false>(f[0], f[1], 0);
      const f32x2 dec = __builtin_amdgcn_cvt_pk_f32_fp8(code2, false);
      // Round the product to fp32 first, then to fp16: the opaque step keeps
      // the compiler from fusing both roundings into one mixed-precision FMA.
      float p0 = dec.x * svf, p1 = dec.y * svf;
      opaque(p0, p1);
      w[e2] = uint32_t(f32_to_f16(p0)) | (uint32_t(f32_to_f16(p1)) << 16);
    }
    *reinterpret_cast<uint4*>(vlow + d * BK + q * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D, int BQ, bool MOM>
__global__ __launch_bounds__(kThreads) void k1_q(PoolArgs a) {
  using BL = BlockLoad<D, BQ>;
  __shared__ double red[BL::RT * D];
  __shared__ float fred[kThreads / 64];
  __shared__ double dred[kThreads / 64];
  const Dims& dm = a.d;
  const int bh = blockIdx.x / dm.Nq, I = blockIdx.x % dm.Nq;
  const int b = bh / dm.H, h = bh % dm.H;
  const int rows = min(BQ, dm.N - I * BQ);
  const int64_t off = (int64_t)b * dm.sb + (int64_t)h * dm.sh + (int64_t)I * BQ * dm.sn;
  unsigned char* ws = a.ws;
  float* qbar = reinterpret_cast<float*>(ws + a.L.qbar) + ((int64_t)bh * dm.Nq + I) * D;
  BL bl;
  double colsum, colsq = 0.0;
  float amax;
  load_block<D, BQ, MOM>(a.q + off, dm.sn, rows, bl, red, colsum, amax, &colsq);
  if (threadIdx.x < D) qbar[threadIdx.x] = static_cast<float>(colsum / static_cast<double>(rows));
  if (MOM) {   // query mean square per dimension and its total
    const int64_t qb = (int64_t)bh * dm.Nq + I;
    const ColMoments cm = col_moments(colsum, colsq, rows);
    if (threadIdx.x < D) reinterpret_cast<float*>(ws + a.L.q2)[qb * D + threadIdx.x] = static_cast<float>(cm.msq);
    const double tot = block_sum_d(threadIdx.x < D ? cm.msq : 0.0, dred);
    if (threadIdx.x == 0) reinterpret_cast<float*>(ws + a.L.m2q)[qb] = static_cast<float>(tot);
  }
  amax = block_max(amax, fred);
  if (threadIdx.x == 0) {
    reinterpret_cast<float*>(ws + a.L.sq)[(int64_t)bh * dm.Nq + I] = scale448(amax);
    reinterpret_cast<float*>(ws + a.L.iq)[(int64_t)bh * dm.Nq + I] = inv448(amax);
  }
}

// MXFP4 copies of K_J and V_J for the SKIM tier (64-key blocks; "Triage":
// skimming a tile in a 4-bit format).  Per key row and 32 channels one E8M0
// scale and 32 E2M1 codes.  K: codes [64][D/2] (channel 2m in the low nibble
// of byte m) and scale bytes [64][D/32], row-major; V: the dequantised values
// fl16(code value * 2^e), transposed [D][64] in vt_pos order like the other
// V operands.  Rows past N are zero (codes 0, scale byte 0).
template <int D>
__global__ __launch_bounds__(kThreads) void k1_mx4(PoolArgs a) {
  constexpr int NB = D / 32;            // scale blocks per row
  __shared__ uint16_t tileV[64 * D];    // dequantised V, fp16 [key][d]
  const Dims& dm = a.d;
  const int bh = blockIdx.x / dm.Nk, J = blockIdx.x % dm.Nk;
  const int b = bh / dm.H, h = bh % dm.H;
  const int rows = min(64, dm.N - J * 64);
  const int64_t off = (int64_t)b * dm.sb + (int64_t)h * dm.sh + (int64_t)J * 64 * dm.sn;
  unsigned char* slab = a.ws + a.L.slab + (int64_t)bh * a.L.sl.bytes;
  unsigned char* k4 = slab + a.L.sl.k4 + (int64_t)J * 64 * (D / 2);
  unsigned char* k4s = slab + a.L.sl.k4s + (int64_t)J * 64 * NB;
  uint16_t* vs = reinterpret_cast<uint16_t*>(slab + a.L.sl.vskim) + (int64_t)J * 64 * D;
  for (int u = threadIdx.x; u < 2 * 64 * NB; u += kThreads) {
    const bool isv = u >= 64 * NB;
    const int w = isv ? u - 64 * NB : u;
    const int r = w / NB, c = w % NB;
    const uint16_t* src = (isv ? a.v : a.k) + off + (int64_t)r * dm.sn + 32 * c;
    float x[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (r < rows) raw = reinterpret_cast<const uint4*>(src)[i];
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float f = __uint_as_float(e & 1 ? (wd[e >> 1] & 0xffff0000u) : (wd[e >> 1] << 16));
        x[8 * i + e] = f;
        amax = __builtin_fmaxf(amax, __builtin_fabsf(f));
      }
    }
    const int ex = mx4_exponent(amax);
    if (!isv) {
      uint32_t pk[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 32; e++) pk[e >> 3] |= e2m1_code(ldexpf(x[e], -ex)) << (4 * (e & 7));
      *reinterpret_cast<uint4*>(k4 + r * (D / 2) + 16 * c) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      k4s[r * NB + c] = static_cast<unsigned char>(ex + 127);
    } else {
#pragma unroll
      for (int e = 0; e < 32; e++)
        tileV[r * D + 32 * c + e] = f32_to_f16(ldexpf(e2m1_value(e2m1_code(ldexpf(x[e], -ex))), ex));
    }
  }
  __syncthreads();
  // element e of stored row d holds key vt_key<64>(e), 8 elements per store
  for (int u = threadIdx.x; u < D * 8; u += kThreads) {
    const int d = u / 8, q = u % 8;
    uint32_t w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; e2++)
      w[e2] = uint32_t(tileV[vt_key<64>(q * 8 + 2 * e2) * D + d]) |
              (uint32_t(tileV[vt_key<64>(q * 8 + 2 * e2 + 1) * D + d]) << 16);
    *reinterpret_cast<uint4*>(vs + d * 64 + q * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D, bool MOM>
hipError_t launch_pool_d(const PoolArgs& a, hipStream_t s) {
  const Dims& d = a.d;
  if (d.Bk == 64)
    hipLaunchKernelGGL((k1_kv<D, 64, MOM>), dim3(d.BH * d.Nk), dim3(kThreads), 0, s, a);
  else if (d.Bk == 16)
    hipLaunchKernelGGL((k1_kv<D, 16, MOM>), dim3(d.BH * d.Nk), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k1_kv<D, 8, MOM>), dim3(d.BH * d.Nk), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d.Bq == 128)
    hipLaunchKernelGGL((k1_q<D, 128, MOM>), dim3(d.BH * d.Nq), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k1_q<D, 64, MOM>), dim3(d.BH * d.Nq), dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || !a.mx4) return e;
  if (d.Bk != 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k1_mx4<D>), dim3(d.BH * d.Nk), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  if (a.moments) return a.d.D == 128 ? launch_pool_d<128, true>(a, s) : launch_pool_d<64, true>(a, s);
  return a.d.D == 128 ? launch_pool_d<128, false>(a, s) : launch_pool_d<64, false>(a, s);
}

}  // namespace tattn
