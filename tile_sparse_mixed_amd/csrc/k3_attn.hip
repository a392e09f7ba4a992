// K3: the fused three-tier attention pass ("Triage": skip / low precision /
// full tiles executed in a single pass; "APT": dual-precision compute units
// and a tile dataflow; "FG-Attn": dense work only on kept tiles).
//
// One workgroup per (b, h, query block I) of BQ = 32 * NW rows; wave w owns
// rows 32w..32w+31.  The workgroup walks the block's compacted list:
//   FULL tiles   K (bf16, the caller's tensor) and V^T (fp16 transposed copy,
//                exact for bf16 values in fp16's normal range): S^T = K Q^T on
//                v_mfma_f32_32x32x16_bf16, O^T += V^T P^T on the fp16 variant
//                (P in [0, 2^8] keeps 3 more mantissa bits than bf16 would),
//   LOW tiles    E4M3 K codes and the fp16 dequantised E4M3 V: S^T on
//                v_mfma_f32_32x32x64_f8f6f4 from the E4M3 Q and K copies, scaled
//                by sq*sk; P.V on the fp16 instruction as for FULL tiles,
//   SKIP chunks  up to 64 skipped key blocks gathered as pseudo-keys kbar_J
//                (a bf16 hi + lo pair, two MFMAs, so the skipped scores keep
//                ~2^-17 precision) with a log2(n_J) bias and values vbar_J
//                (fp16): one score per
//                skipped block weighted by n_J ("Triage": block means),
// keeping an online softmax per query row in base 2.  Tiles stream through
// two LDS stages (register-staged global loads overlap the current tile's
// math).  S^T puts one query per lane, so row statistics need only the lane
// pair (l, l^32).
//
// Running state per lane (query row): m (base-2 reference), l (sum of the
// rounded weights the MFMAs multiply, relative to 2^m) and the O^T
// accumulator.  m is raised only when a tile's max exceeds it by more than 8
// (weights stay <= 2^8), so most tiles skip the accumulator rescale.
#include "tattn_device.hpp"
#include "tattn_internal.hpp"

namespace tattn {
namespace {

constexpr float kLazy = 8.0f;     // raise m only when a tile max exceeds it by this much (log2)

template <int D, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BQ = NW * 32;
  static constexpr int KCH = D / 8;               // 16-byte chunks of a bf16 K row
  static constexpr int STAGE = 384 * D;           // bytes of one LDS stage: K | V^T | K lo (skip chunks)
  static constexpr int KPT = (64 * KCH) / NT;     // bf16 K chunks per thread
  static constexpr int VPT = (D * 8) / NT;        // bf16 V^T chunks per thread
  static constexpr int K8PT = (64 * D / 16) / NT; // fp8 K chunks per thread
  static constexpr int SREG = 2 * KPT + VPT;      // a skip chunk stages K hi, V and K lo
  static_assert((64 * KCH) % NT == 0 && (D * 8) % NT == 0, "tile split");
  static_assert((64 * D / 16) % NT == 0, "fp8 tile split");
};

// swizzled byte offsets inside a stage
template <int D>
__device__ inline int offK(int row, int ch) { return row * (2 * D) + ((ch ^ (row & 7)) << 4); }
__device__ inline int offV(int d, int ch) { return d * 128 + ((ch ^ (d & 7)) << 4); }
template <int D>
__device__ inline int offK8(int row, int ch) {
  return D == 128 ? row * 128 + ((ch ^ (row & 7)) << 4) : row * 64 + ((ch ^ ((row >> 1) & 3)) << 4);
}

enum StepKind { kFull = 0, kLow = 1, kSkip = 2 };

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void k3_attn(AttnArgs a) {
  using C = Cfg<D, NW>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::STAGE];
  __shared__ float sbias[2][64];

  const Dims& dm = a.d;
  // ---- XCD-aware work mapping: consecutive workgroups go round-robin over
  // the 8 XCDs; give each XCD a contiguous range of (b, h, I) so that the
  // query blocks of a head share that XCD's L2.
  const int G = dm.BH * dm.Nq;
  int w_item;
  {
    const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
    const int q = G >> 3, r = G & 7;
    w_item = xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
  }
  const int bh = w_item / dm.Nq, I = w_item % dm.Nq;
  const int bidx = bh / dm.H, hidx = bh % dm.H;
  const int64_t toff = (int64_t)bidx * dm.sb + (int64_t)hidx * dm.sh;
  const int64_t row = (int64_t)bh * dm.Nq + I;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, lh = lane >> 5;   // query column inside the wave, lane half

  unsigned char* ws = a.ws;
  const int* counts = reinterpret_cast<const int*>(ws + a.L.counts) + row * 4;
  const int nF = counts[0], nL = counts[1], nS = counts[2];
  const int16_t* list = reinterpret_cast<const int16_t*>(ws + a.L.lists) + row * dm.Nk;
  const int nSc = (nS + 63) >> 6;
  const int nSteps = nF + nL + nSc;

  const uint16_t* kin = a.k + toff;
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(ws + a.L.vt) + (int64_t)bh * dm.Nk * 64 * D;  // fp16 bits
  const unsigned char* k8 = ws + a.L.k8 + (int64_t)bh * dm.Nk * 64 * D;
  const uint16_t* vlow = reinterpret_cast<const uint16_t*>(ws + a.L.vlow) + (int64_t)bh * dm.Nk * 64 * D;
  const uint16_t* kb16 = reinterpret_cast<const uint16_t*>(ws + a.L.kbar16) + (int64_t)bh * dm.Nk * D;
  const uint16_t* kblo = reinterpret_cast<const uint16_t*>(ws + a.L.kbarlo) + (int64_t)bh * dm.Nk * D;
  const uint16_t* vb16 = reinterpret_cast<const uint16_t*>(ws + a.L.vbar16) + (int64_t)bh * dm.Nk * D;
  const float* skp = reinterpret_cast<const float*>(ws + a.L.sk) + (int64_t)bh * dm.Nk;

  // ---- Q rows of this wave as bf16 B operands: lane (ln, lh) holds
  // q[row][16c + 8lh .. +8] for chunk c.
  const int qrow = I * C::BQ + wave * 32 + ln;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; c++) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qrow < dm.N) v = *reinterpret_cast<const uint4*>(a.q + toff + (int64_t)qrow * dm.sn + 16 * c + 8 * lh);
    qreg[c] = __builtin_bit_cast(bf16x8, v);
  }
  // fp8 copy for LOW tiles: 32 bytes per instruction i = chunks 4i..4i+3
  i32x8 q8reg[D / 64];
  const float sq = reinterpret_cast<const float*>(ws + a.L.sq)[row];
  if (nL > 0) {
    const float iq = reinterpret_cast<const float*>(ws + a.L.iq)[row];
#pragma unroll
    for (int i = 0; i < D / 64; i++) {
#pragma unroll
      for (int cc = 0; cc < 4; cc++) {
        const uint4 raw = __builtin_bit_cast(uint4, qreg[4 * i + cc]);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
        int lo = 0, hi = 0;
        lo = cvt_fp8x2<false>(__uint_as_float(w4[0] << 16) * iq, __uint_as_float(w4[0] & 0xffff0000u) * iq, lo);
        lo = cvt_fp8x2<true>(__uint_as_float(w4[1] << 16) * iq, __uint_as_float(w4[1] & 0xffff0000u) * iq, lo);
        hi = cvt_fp8x2<false>(__uint_as_float(w4[2] << 16) * iq, __uint_as_float(w4[2] & 0xffff0000u) * iq, hi);
        hi = cvt_fp8x2<true>(__uint_as_float(w4[3] << 16) * iq, __uint_as_float(w4[3] & 0xffff0000u) * iq, hi);
        q8reg[i][2 * cc] = lo;
        q8reg[i][2 * cc + 1] = hi;
      }
    }
  }

  // ---- staging: global -> registers -> LDS
  uint4 stg[C::SREG];
  float bias_stg = -INFINITY;

  auto step_kind = [&](int t) { return t < nF ? kFull : (t < nF + nL ? kLow : kSkip); };

  auto stage_load = [&](int t) {
    const int kind = step_kind(t);
    if (kind == kFull) {
      const int J = list[t];
      const uint16_t* vtile = vt + (int64_t)J * 64 * D;
#pragma unroll
      for (int i = 0; i < C::KPT; i++) {
        const int u = tid + i * C::NT, r = u / C::KCH, ch = u % C::KCH;
        const int g = J * 64 + r;
        stg[i] = g < dm.N ? *reinterpret_cast<const uint4*>(kin + (int64_t)g * dm.sn + ch * 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < C::VPT; i++) {
        const int u = tid + i * C::NT;
        stg[C::KPT + i] = *reinterpret_cast<const uint4*>(vtile + u * 8);
      }
    } else if (kind == kLow) {
      const int J = list[t];
      const unsigned char* ktile = k8 + (int64_t)J * 64 * D;
      const uint16_t* vtile = vlow + (int64_t)J * 64 * D;
#pragma unroll
      for (int i = 0; i < C::K8PT; i++) stg[i] = *reinterpret_cast<const uint4*>(ktile + (tid + i * C::NT) * 16);
#pragma unroll
      for (int i = 0; i < C::VPT; i++) stg[C::K8PT + i] = *reinterpret_cast<const uint4*>(vtile + (tid + i * C::NT) * 8);
    } else {
      const int base = nF + nL + ((t - nF - nL) << 6);
      const int cnt = min(64, nF + nL + nS - base);
#pragma unroll
      for (int i = 0; i < C::KPT; i++) {
        const int u = tid + i * C::NT, s = u / C::KCH, ch = u % C::KCH;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0), kl = make_uint4(0, 0, 0, 0);
        if (s < cnt) {
          const int J = list[base + s];
          kv = *reinterpret_cast<const uint4*>(kb16 + (int64_t)J * D + ch * 8);
          vv = *reinterpret_cast<const uint4*>(vb16 + (int64_t)J * D + ch * 8);
          kl = *reinterpret_cast<const uint4*>(kblo + (int64_t)J * D + ch * 8);
        }
        stg[i] = kv;
        stg[C::KPT + i] = vv;   // KPT == VPT here (both 8D/NT)
        stg[C::KPT + C::VPT + i] = kl;
      }
      if (tid < 64) {
        bias_stg = -INFINITY;
        if (tid < cnt) {
          const int J = list[base + tid];
          bias_stg = __log2f(static_cast<float>(min(64, dm.N - J * 64)));
        }
      }
    }
  };

  auto stage_store = [&](int t, int buf) {
    unsigned char* st = smem + buf * C::STAGE;
    const int kind = step_kind(t);
    if (kind == kFull || kind == kSkip) {
#pragma unroll
      for (int i = 0; i < C::KPT; i++) {
        const int u = tid + i * C::NT, r = u / C::KCH, ch = u % C::KCH;
        *reinterpret_cast<uint4*>(st + offK<D>(r, ch)) = stg[i];
      }
      unsigned char* sv = st + 128 * D;
      if (kind == kFull) {
#pragma unroll
        for (int i = 0; i < C::VPT; i++) {
          const int u = tid + i * C::NT, d = u >> 3, ch = u & 7;
          *reinterpret_cast<uint4*>(sv + offV(d, ch)) = stg[C::KPT + i];
        }
      } else {
        // gathered vbar rows (fp16), written transposed: element (key s, d) -> row d, vt_pos(s)
#pragma unroll
        for (int i = 0; i < C::KPT; i++) {
          const int u = tid + i * C::NT, s = u / C::KCH, ch = u % C::KCH;
          const int pos = vt_pos(s), q = pos >> 3, e = pos & 7;
          const uint32_t w4[4] = {stg[C::KPT + i].x, stg[C::KPT + i].y, stg[C::KPT + i].z, stg[C::KPT + i].w};
#pragma unroll
          for (int z = 0; z < 8; z++) {
            const int d = ch * 8 + z;
            const uint16_t val = static_cast<uint16_t>(z & 1 ? (w4[z >> 1] >> 16) : (w4[z >> 1] & 0xffffu));
            *reinterpret_cast<uint16_t*>(sv + offV(d, q) + 2 * e) = val;
          }
        }
#pragma unroll
        for (int i = 0; i < C::KPT; i++) {
          const int u = tid + i * C::NT, r = u / C::KCH, ch = u % C::KCH;
          *reinterpret_cast<uint4*>(st + 256 * D + offK<D>(r, ch)) = stg[C::KPT + C::VPT + i];
        }
        if (tid < 64) sbias[buf][tid] = bias_stg;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::K8PT; i++) {
        const int u = tid + i * C::NT;
        const int r = u / (D / 16), ch = u % (D / 16);
        *reinterpret_cast<uint4*>(st + offK8<D>(r, ch)) = stg[i];
      }
#pragma unroll
      for (int i = 0; i < C::VPT; i++) {
        const int u = tid + i * C::NT, d = u >> 3, ch = u & 7;
        *reinterpret_cast<uint4*>(st + 128 * D + offV(d, ch)) = stg[C::K8PT + i];
      }
    }
  };

  // ---- online-softmax state
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; db++) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float cF = kLog2e / __builtin_sqrtf(static_cast<float>(D));

  // Raise the reference max of the lanes whose tile max exceeds it by more
  // than kLazy; rescale their l and accumulator.
  auto raise_max = [&](float tm) {
    const bool need = tm > m_run + kLazy;
    if (__ballot(need)) {
      const float mn = need ? tm : m_run;
      const float al = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
      l_run *= al;
#pragma unroll
      for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[db][r] *= al;
      m_run = mn;
    }
  };

  if (nSteps > 0) {
    stage_load(0);
    stage_store(0, 0);
  }
  __syncthreads();

  for (int t = 0; t < nSteps; t++) {
    const int buf = t & 1;
    if (t + 1 < nSteps) stage_load(t + 1);
    const unsigned char* st = smem + buf * C::STAGE;
    const int kind = step_kind(t);
    f32x16 s[2] = {f32x16{}, f32x16{}};

    // ---- scores S^T = K Q^T for the 64 keys of the step
    if (kind == kLow) {
#pragma unroll
      for (int i = 0; i < D / 64; i++) {
#pragma unroll
        for (int b = 0; b < 2; b++) {
          const int r = 32 * b + ln;
          const int ch0 = (D == 128 ? 4 * i : 0) + 2 * lh;
          const uint4 lo = *reinterpret_cast<const uint4*>(st + offK8<D>(r, ch0));
          const uint4 hi = *reinterpret_cast<const uint4*>(st + offK8<D>(r, ch0 + 1));
          const i32x8 av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, q8reg[i], s[b], 0, 0, 0, 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < D / 16; c++) {
#pragma unroll
        for (int b = 0; b < 2; b++) {
          const int r = 32 * b + ln;
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(st + offK<D>(r, 2 * c + lh));
          s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[c], s[b], 0, 0, 0);
        }
      }
      if (kind == kSkip) {   // low half of the pooled keys
#pragma unroll
        for (int c = 0; c < D / 16; c++) {
#pragma unroll
          for (int b = 0; b < 2; b++) {
            const int r = 32 * b + ln;
            const bf16x8 av = *reinterpret_cast<const bf16x8*>(st + 256 * D + offK<D>(r, 2 * c + lh));
            s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[c], s[b], 0, 0, 0);
          }
        }
      }
    }

    // ---- online softmax: x in base-2 units
    float x[32];
    float tmax = -INFINITY;
    if (kind == kSkip) {
      const float* bs = sbias[buf];
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float4 bb = *reinterpret_cast<const float4*>(bs + 32 * b + 8 * j + 4 * lh);
          const float bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float v = __builtin_fmaf(s[b][4 * j + i], cF, bv[i]);
            x[16 * b + 4 * j + i] = v;
            tmax = __builtin_fmaxf(tmax, v);
          }
        }
    } else {
      const int J = list[t];
      const int nvalid = min(64, dm.N - J * 64);
      const float c = kind == kLow ? sq * skp[J] * cF : cF;
#pragma unroll
      for (int b = 0; b < 2; b++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int key = 32 * b + 8 * (r >> 2) + 4 * lh + (r & 3);
          const float v = key < nvalid ? s[b][r] * c : -INFINITY;
          x[16 * b + r] = v;
          tmax = __builtin_fmaxf(tmax, v);
        }
    }
    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    raise_max(tmax);
    f16x8 pb[4];
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int tt = 0; tt < 8; tt++)
        pb[cc][tt] = static_cast<_Float16>(__builtin_amdgcn_exp2f(x[8 * cc + tt] - m_run));
    // l sums exactly the rounded weights that enter P.V
    float psum = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int tt = 0; tt < 8; tt++) psum += static_cast<float>(pb[cc][tt]);
    l_run += psum;

    // ---- O^T += V^T P^T (fp16 values: V, the low tier's V, or the skipped blocks' means)
    const unsigned char* sv = st + 128 * D;
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {
#pragma unroll
      for (int db = 0; db < D / 32; db++) {
        const int d = 32 * db + ln;
        const f16x8 av = *reinterpret_cast<const f16x8*>(sv + offV(d, 2 * cc + lh));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[cc], acc[db], 0, 0, 0);
      }
    }

    if (t + 1 < nSteps) stage_store(t + 1, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l
  const float L = l_run + __shfl_xor(l_run, 32, 64);
  const float scale = 1.0f / L;
  if (qrow < dm.N) {
    if (a.out_fp32) {
      float* o = reinterpret_cast<float*>(a.o) + toff + (int64_t)qrow * dm.sn;
#pragma unroll
      for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int d0 = 32 * db + 8 * j + 4 * lh;
          *reinterpret_cast<float4*>(o + d0) = make_float4(acc[db][4 * j] * scale, acc[db][4 * j + 1] * scale,
                                                           acc[db][4 * j + 2] * scale, acc[db][4 * j + 3] * scale);
        }
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(a.o) + toff + (int64_t)qrow * dm.sn;
#pragma unroll
      for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int d0 = 32 * db + 8 * j + 4 * lh;
          const uint32_t lo = f32_to_bf16(acc[db][4 * j] * scale) | (uint32_t(f32_to_bf16(acc[db][4 * j + 1] * scale)) << 16);
          const uint32_t hi = f32_to_bf16(acc[db][4 * j + 2] * scale) | (uint32_t(f32_to_bf16(acc[db][4 * j + 3] * scale)) << 16);
          *reinterpret_cast<uint2*>(o + d0) = make_uint2(lo, hi);
        }
    }
  }
}

template <int D, int NW>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k3_attn<D, NW>), dim3(a.d.BH * a.d.Nq), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int D = a.d.D, BQ = a.d.Bq;
  if (D == 128 && BQ == 128) return launch_one<128, 4>(a, s);
  if (D == 128 && BQ == 64) return launch_one<128, 2>(a, s);
  if (D == 64 && BQ == 128) return launch_one<64, 4>(a, s);
  if (D == 64 && BQ == 64) return launch_one<64, 2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace tattn
