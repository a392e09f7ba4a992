// K2: block router, tier assignment and tile-list compaction.
//
// K2a  S_IJ = <qbar_I, kbar_J> / sqrt(d) + ln n_J in float64, tiled 64 query
//      blocks x 64 key blocks per workgroup through LDS ("APT": attention
//      probability of the block as the importance metric; the ln n_J term
//      weights a key block by its real size).
// K2b  per query block I: p_IJ = softmax_J(S_IJ) (float64), then the tier map:
//        THRESHOLD  FULL if p >= tau_hi, LOW if p >= tau_lo, SKIM if p >=
//                   tau_skim > 0 ("Triage": the 4-bit skim tier), else SKIP;
//                   then an optional top-k by (p desc, J asc) ("APT": dual
//                   thresholds; "HierPAS": top-k),
//        ADAPTIVE   k_h from the entropy of p on sampled rows (K2e), then the top
//                   ceil(full_frac*k_h) tiles FULL, the rest of the top k_h LOW
//                   ("HierPAS": sampling-based entropy, head-wise retention),
//        ALL_FULL   every tile FULL,
//        PRICE      per tile the tier with the least predicted error (from
//                   block second moments, K2a's spread product) plus price x
//                   work, SKIM among the choices with tau_skim > 0
//                   ("Triage": error-predicting router, one price);
//      diagonal tiles forced FULL; then a stable compaction into
//      [FULL asc | LOW asc | SKIM asc | SKIP asc] with wavefront ballots.
// K2c  compaction only, for a tier map supplied by the caller.
// K2d  the order in which the fused kernel takes its rows (longest last rows first).
// Ranks and cuts use exact comparisons of the float64 p values.
#include "tattn_device.hpp"
#include "tattn_internal.hpp"

namespace tattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRouterMaxNk = 4096;

// ------------------------------------------------------------------ K2a
// SPREAD: the same product over the price router's second moments, the
// within-tile score spread s2_IJ = sum_c q2_I,c kvar_J,c / d.
template <int D, bool SPREAD>
__global__ __launch_bounds__(kThreads) void k2a_scores(RouterArgs a) {
  // 64 query blocks x 64 key blocks per workgroup; each thread owns a 4 x 4
  // block of S.  The operands pass through LDS as float64, 16 values of d at
  // a time, so the inner loop is 4 LDS reads per 16 FMAs and no conversions.
  constexpr int DC = 16;
  __shared__ __attribute__((aligned(16))) double qs[DC][64];   // qbar chunk, [d][row]
  __shared__ __attribute__((aligned(16))) double ks[DC][64];   // kbar chunk, [d][J]
  const Dims& dm = a.d;
  const int bh = blockIdx.z;
  const int I0 = blockIdx.y * 64, J0 = blockIdx.x * 64;
  const float* qbar = reinterpret_cast<const float*>(a.ws + (SPREAD ? a.L.q2 : a.L.qbar)) + (int64_t)bh * dm.Nq * D;
  const float* kbar = reinterpret_cast<const float*>(a.ws + (SPREAD ? a.L.kvar : a.L.kbar)) + (int64_t)bh * dm.Nk * D;
  const int t = threadIdx.x;
  const int rg = t / 16, jg = t % 16;   // rows 4rg..4rg+3, key blocks 4jg..4jg+3
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = 0.0;
  for (int c0 = 0; c0 < D; c0 += DC) {
    // 64 rows x 16 d of each operand: thread t loads row t / 4, d 4(t % 4) .. +3
    {
      const int r = t >> 2, c = 4 * (t & 3);
      float4 qv = make_float4(0.f, 0.f, 0.f, 0.f), kv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (I0 + r < dm.Nq) qv = *reinterpret_cast<const float4*>(qbar + (int64_t)(I0 + r) * D + c0 + c);
      if (J0 + r < dm.Nk) kv = *reinterpret_cast<const float4*>(kbar + (int64_t)(J0 + r) * D + c0 + c);
      qs[c][r] = qv.x; qs[c + 1][r] = qv.y; qs[c + 2][r] = qv.z; qs[c + 3][r] = qv.w;
      ks[c][r] = kv.x; ks[c + 1][r] = kv.y; ks[c + 2][r] = kv.z; ks[c + 3][r] = kv.w;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < DC; c++) {
      const double2 q01 = *reinterpret_cast<const double2*>(&qs[c][4 * rg]);
      const double2 q23 = *reinterpret_cast<const double2*>(&qs[c][4 * rg + 2]);
      const double2 k01 = *reinterpret_cast<const double2*>(&ks[c][4 * jg]);
      const double2 k23 = *reinterpret_cast<const double2*>(&ks[c][4 * jg + 2]);
      const double q[4] = {q01.x, q01.y, q23.x, q23.y};
      const double k[4] = {k01.x, k01.y, k23.x, k23.y};
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = fma(q[i], k[j], acc[i][j]);
    }
    __syncthreads();
  }
  double* S = reinterpret_cast<double*>(a.ws + (SPREAD ? a.L.s2 : a.L.S)) + (int64_t)bh * dm.Nq * dm.Nk;
  // 1/d is exact for d a power of two, so the spread is acc / d exactly
  const double isd = SPREAD ? 1.0 / static_cast<double>(D) : 1.0 / sqrt(static_cast<double>(D));
  const double lg_full = SPREAD ? 0.0 : log(static_cast<double>(dm.Bk));
  const double lg_last = SPREAD ? 0.0 : log(static_cast<double>(dm.N - (dm.Nk - 1) * dm.Bk));
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int I = I0 + 4 * rg + i;
    if (I >= dm.Nq) continue;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int J = J0 + 4 * jg + j;
      if (J >= dm.Nk) continue;
      S[(int64_t)I * dm.Nk + J] = fma(acc[i][j], isd, J == dm.Nk - 1 ? lg_last : lg_full);
    }
  }
}

// ------------------------------------------------------------------ block reductions
struct Red {
  double d[kWaves];
  int i[kWaves * 8];
  uint64_t u[kWaves];
  // radix-select digit histogram, one per wave: a pair of waves shares a word,
  // 16 bits each (a wave counts at most kMaxNk / kWaves values)
  int hist[kWaves / 2][256];
  int sel[3];      // selected digit, count of candidates above it, candidates holding it
};

__device__ double block_max_d(double v, Red& r) {
  v = wave_max_d(v);
  if ((threadIdx.x & 63) == 0) r.d[threadIdx.x >> 6] = v;
  __syncthreads();
  double m = r.d[0];
#pragma unroll
  for (int w = 1; w < kWaves; w++) m = fmax(m, r.d[w]);
  __syncthreads();
  return m;
}
__device__ double block_sum_d(double v, Red& r) {
  v = wave_sum_d(v);
  if ((threadIdx.x & 63) == 0) r.d[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = r.d[0];
#pragma unroll
  for (int w = 1; w < kWaves; w++) s += r.d[w];
  __syncthreads();
  return s;
}
__device__ int block_sum_i(int v, Red& r) {
  v = wave_sum_i(v);
  if ((threadIdx.x & 63) == 0) r.i[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kWaves; w++) s += r.i[w];
  __syncthreads();
  return s;
}

// Largest (MAX) or smallest bit pattern among the pv[J] at or above `floor`
// whose bits match `prefix` under `mask`; at least one does.
template <bool MAX>
__device__ uint64_t block_extreme_bits(const double* pv, int n, uint64_t prefix, uint64_t mask, uint64_t floor,
                                       Red& r) {
  uint64_t v = MAX ? 0ull : ~0ull;
  for (int J = threadIdx.x; J < n; J += kThreads) {
    const uint64_t b = (uint64_t)__double_as_longlong(pv[J]);
    if (b >= floor && (b & mask) == prefix) v = MAX ? (b > v ? b : v) : (b < v ? b : v);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t x = __shfl_xor(v, o, 64);
    v = MAX ? (x > v ? x : v) : (x < v ? x : v);
  }
  if ((threadIdx.x & 63) == 0) r.u[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t e = r.u[0];
#pragma unroll
  for (int w = 1; w < kWaves; w++) e = MAX ? (r.u[w] > e ? r.u[w] : e) : (r.u[w] < e ? r.u[w] : e);
  __syncthreads();
  return e;
}

// Bits of the k-th largest value (1 <= k <= n) among the non-negative doubles
// pv[0..n).  Non-negative doubles order like their bit patterns, so this is a
// radix select from the top byte down: per byte, a histogram of that byte over
// the values that match the bytes chosen so far, then the byte at which the
// count from the top reaches the remaining rank.  Once that rank is the first
// or the last of the values still matching, one max or min reduction ends the
// select; on continuous data this happens after two or three bytes.
// (Measured against 11-bit digits: 8-bit digits are faster; fewer bins to
// clear and scan per pass outweigh the contention of the top byte.)
// Values below the bit pattern `floor` are left out; the caller guarantees
// that the k-th largest is at or above it (0: none left out).
__device__ uint64_t kth_largest_bits(const double* pv, int n, int k, uint64_t floor, Red& r) {
  uint64_t prefix = 0, mask = 0;
  int kk = k;   // rank of the wanted value among the values matching `prefix`
  const int lane = threadIdx.x & 63;
  for (int sh = 56; sh >= 0; sh -= 8) {
    constexpr int bins = 256;
    for (int i = threadIdx.x; i < bins * (kWaves / 2); i += kThreads) (&r.hist[0][0])[i] = 0;
    __syncthreads();
    {
      int* hw = r.hist[threadIdx.x >> 7];
      const int one = 1 << (((threadIdx.x >> 6) & 1) * 16);
      for (int J = threadIdx.x; J < n; J += kThreads) {
        const uint64_t b = (uint64_t)__double_as_longlong(pv[J]);
        if (b >= floor && (b & mask) == prefix) atomicAdd(&hw[(b >> sh) & (bins - 1)], one);
      }
    }
    __syncthreads();
    if (threadIdx.x < bins) {   // fold the per-wave counts into one histogram
      int c = 0;
#pragma unroll
      for (int ww = 0; ww < kWaves / 2; ww++) c += (r.hist[ww][threadIdx.x] & 0xffff) + (r.hist[ww][threadIdx.x] >> 16);
      r.hist[0][threadIdx.x] = c;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns digits 255 - 4l .. 252 - 4l (descending);
      // inclusive scan of the lane totals from the top digit down
      const int w = bins >> 6;
      int tot = 0;
      for (int j = 0; j < w; j++) tot += r.hist[0][bins - 1 - lane * w - j];
      int cum = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int up = __shfl_up(cum, o, 64);
        if (lane >= o) cum += up;
      }
      const uint64_t hit = __ballot(cum >= kk);
      const int L = __ffsll((long long)hit) - 1;   // first lane whose range reaches kk
      if (lane == L) {
        int above = cum - tot;
        for (int j = 0; j < w; j++) {
          const int c = r.hist[0][bins - 1 - lane * w - j];
          if (above + c >= kk) {
            r.sel[0] = bins - 1 - lane * w - j;
            r.sel[1] = above;
            r.sel[2] = c;
            break;
          }
          above += c;
        }
      }
    }
    __syncthreads();
    prefix |= (uint64_t)r.sel[0] << sh;
    mask |= (uint64_t)(bins - 1) << sh;
    kk -= r.sel[1];
    const int cand = r.sel[2];
    __syncthreads();
    if (sh > 0 && kk == 1) return block_extreme_bits<true>(pv, n, prefix, mask, floor, r);
    if (sh > 0 && kk == cand) return block_extreme_bits<false>(pv, n, prefix, mask, floor, r);
  }
  return prefix;
}

// rank(J) < k  <=>  p_J > x_k  or  (p_J == x_k and J is among the first `need`
// tiles equal to x_k in ascending J), need = k - #{p > x_k}.  Calls
// mark(J, rank(J) < k) once for every tile; a barrier follows.  `floor`: a
// bit pattern known to be at or below x_k (the select then skips the values
// under it); returns x_k's bits (0 when k <= 0 or k >= n).
template <class Mark>
__device__ uint64_t mark_top_k(const double* pv, int n, int k, Mark mark, Red& r, uint64_t floor = 0) {
  if (k >= n || k <= 0) {
    for (int J = threadIdx.x; J < n; J += kThreads) mark(J, k > 0);
    __syncthreads();
    return 0;
  }
  const uint64_t xb = kth_largest_bits(pv, n, k, floor, r);
  int ge = 0;   // #{p > x} in the low 16 bits, #{p == x} above (n <= 4096)
  for (int J = threadIdx.x; J < n; J += kThreads) {
    const uint64_t b = (uint64_t)__double_as_longlong(pv[J]);
    ge += (b > xb) + ((b == xb) << 16);
  }
  ge = block_sum_i(ge, r);
  const int need = k - (ge & 0xffff);
  if (need == (ge >> 16)) {   // every tile equal to x is kept: no ordering among them needed
    for (int J = threadIdx.x; J < n; J += kThreads) mark(J, (uint64_t)__double_as_longlong(pv[J]) >= xb);
    __syncthreads();
    return xb;
  }
  int base = 0;   // equal-to-x tiles already seen in earlier chunks
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int J0 = 0; J0 < n; J0 += kThreads) {
    const int J = J0 + threadIdx.x;
    const uint64_t b = J < n ? (uint64_t)__double_as_longlong(pv[J]) : 0;
    const bool eq = J < n && b == xb;
    const uint64_t bal = __ballot(eq);
    const int pre = __popcll(bal & ((1ull << lane) - 1));
    if (lane == 0) r.i[w] = __popcll(bal);
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ww++) {
      if (ww < w) woff += r.i[ww];
      tot += r.i[ww];
    }
    if (J < n) mark(J, (b > xb) || (eq && base + woff + pre < need));
    base += tot;
    __syncthreads();
  }
  return xb;
}

// Diagonal tiles of query block I: key blocks whose token range meets I's.
__device__ inline void diag_range(const Dims& dm, int I, int& j0, int& j1) {
  const int r0 = I * dm.Bq, r1 = min(dm.N, (I + 1) * dm.Bq);
  j0 = r0 / dm.Bk;
  j1 = (r1 - 1) / dm.Bk;
}

// Stable compaction of the tier row `tr` (in LDS) into lists [FULL | LOW |
// SKIM | SKIP] and counts = (n_full, n_low, n_skip, steps): steps is the
// number of steps the fused kernel takes for the row, ceil(nF/G) + ceil(nL/G)
// + ceil(nK/G) + 2 x (chunks of 64 key blocks holding a skipped block), G =
// 64 / Bk key blocks per step, nK the SKIM count; it orders the fused
// kernel's work.
__device__ void compact_row(const unsigned char* tr, int n, int bk, int16_t* list, int* counts, Red& r) {
  // each wave owns a run of whole 64-tile chunks: it counts its tiers, one
  // barrier publishes the per-wave counts, then it writes its run in order
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nch = (n + 63) / 64, cpw = (nch + kWaves - 1) / kWaves;
  const int c0 = w * cpw, c1 = min(nch, c0 + cpw);
  const uint64_t below = (1ull << lane) - 1;
  int cnt[4] = {0, 0, 0, 0}, sch = 0;   // indexed by tier value
  for (int c = c0; c < c1; c++) {
    const int J = c * 64 + lane;
    const int tv = J < n ? tr[J] : -1;
#pragma unroll
    for (int T = 0; T < 4; T++) {
      const uint64_t bal = __ballot(tv == T);
      cnt[T] += __popcll(bal);
      if (T == TATTN_SKIP) sch += bal != 0;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int T = 0; T < 4; T++) r.i[w * 8 + T] = cnt[T];
    r.i[w * 8 + 4] = sch;
  }
  __syncthreads();
  int woff[4] = {0, 0, 0, 0}, tot[4] = {0, 0, 0, 0}, snc = 0;
#pragma unroll
  for (int ww = 0; ww < kWaves; ww++) {
#pragma unroll
    for (int T = 0; T < 4; T++) {
      if (ww < w) woff[T] += r.i[ww * 8 + T];
      tot[T] += r.i[ww * 8 + T];
    }
    snc += r.i[ww * 8 + 4];
  }
  const int nF = tot[TATTN_FULL], nL = tot[TATTN_LOW], nS = tot[TATTN_SKIP], nK = tot[TATTN_SKIM];
  if (threadIdx.x == 0) {
    const int G = 64 / bk;
    counts[0] = nF;
    counts[1] = nL;
    counts[2] = nS;
    counts[3] = (nF + G - 1) / G + (nL + G - 1) / G + (nK + G - 1) / G + 2 * snc;
  }
  int base[4];   // indexed by tier value
  base[TATTN_FULL] = woff[TATTN_FULL];
  base[TATTN_LOW] = nF + woff[TATTN_LOW];
  base[TATTN_SKIM] = nF + nL + woff[TATTN_SKIM];
  base[TATTN_SKIP] = nF + nL + nK + woff[TATTN_SKIP];
  for (int c = c0; c < c1; c++) {
    const int J = c * 64 + lane;
    const int tv = J < n ? tr[J] : -1;
#pragma unroll
    for (int T = 0; T < 4; T++) {
      const uint64_t bal = __ballot(tv == T);
      if (tv == T) list[base[T] + __popcll(bal & below)] = static_cast<int16_t>(J);
      base[T] += __popcll(bal);
    }
  }
  __syncthreads();   // r.i is free again
}

// ------------------------------------------------------------------ price router
// Per-tile error model of the price router ("Triage": a tile's error under
// each tier predicted from block statistics; one price trades error against
// work).  Evaluated with every operation rounded on its own (no fused
// multiply-add), in float64.
constexpr double kE4m3U = 0.0625;   // 2^-4: largest relative rounding error of an E4M3 normal value
constexpr double kE2m1U = 0.25;     // 2^-2: the same for an E2M1 (MXFP4) normal value

// log-mass gain of a tile over its pooled estimate: lognormal mean s2/2 up to
// s2 = 2 ln n, beyond it the largest of n scores dominates
__device__ inline double spread_gain(double s2, double lnn) {
#pragma clang fp contract(off)
  return s2 <= 2.0 * lnn ? 0.5 * s2 : sqrt(2.0 * s2 * lnn) - lnn;
}

struct PriceTile {
  double s2, n, vnorm, vvar, m2v, sl2, sk2;   // sk2: the score-noise variance of MXFP4 copies
};
// the tier with the least p~ * error + price * work; ties to the cheaper tier
// (SKIP < SKIM < LOW < FULL in work); SKIM competes only with `skim`
__device__ inline unsigned char price_tier(const PriceTile& x, double pt, double price, double cost_skip, bool skim) {
#pragma clang fp contract(off)
  const double neff = fmax(1.0, x.n * exp(-x.s2));
  const double lnn = log(x.n);
  const double g = spread_gain(x.s2, lnn);
  const double eS = x.vnorm * (-expm1(-g)) + sqrt(x.vvar * fmax(0.0, 1.0 / neff - 1.0 / x.n));
  const double eL = x.vnorm * expm1(0.5 * x.sl2) +
                    (sqrt(x.vvar * expm1(x.sl2)) + kE4m3U * sqrt(x.m2v / 3.0)) / sqrt(neff);
  const double oS = pt * eS + price * cost_skip;
  const double oL = pt * eL + price * 0.5;
  const double oF = price * 1.0;
  unsigned char t = TATTN_SKIP;
  double best = oS;
  if (skim) {
    const double eK = x.vnorm * expm1(0.5 * x.sk2) +
                      (sqrt(x.vvar * expm1(x.sk2)) + kE4m3U * sqrt(x.m2v / 3.0)) / sqrt(neff);
    const double oK = pt * eK + price * 0.375;
    if (oK < best) {
      t = TATTN_SKIM;
      best = oK;
    }
  }
  if (oL < best) {
    t = TATTN_LOW;
    best = oL;
  }
  if (oF < best) t = TATTN_FULL;
  return t;
}

// The price router's tier row: p is exported; the decision uses the shares
// corrected by each tile's spread gain, p~ = softmax_J(S + g).  pv holds p on
// entry and is reused for p~.
__device__ void price_row(const RouterArgs& a, int bh, int64_t row, const double* S, double* pv,
                                       unsigned char* tr, float* pout, Red& r) {
  const Dims& dm = a.d;
  const int n = dm.Nk;
  // p is exported; the decision uses the shares corrected by each tile's
  // spread gain, p~ = softmax_J(S + g)
  const double* s2r = reinterpret_cast<const double*>(a.ws + a.L.s2) + row * n;
  const float* m2k = reinterpret_cast<const float*>(a.ws + a.L.m2k) + (int64_t)bh * n;
  const float* vvar = reinterpret_cast<const float*>(a.ws + a.L.vvar) + (int64_t)bh * n;
  const float* m2v = reinterpret_cast<const float*>(a.ws + a.L.m2v) + (int64_t)bh * n;
  const float* vnorm = reinterpret_cast<const float*>(a.ws + a.L.vnorm) + (int64_t)bh * n;
  const double m2q = reinterpret_cast<const float*>(a.ws + a.L.m2q)[row];
  const double nfull = dm.Bk, nlast = dm.N - (dm.Nk - 1) * dm.Bk;
  const double lnf = log(nfull), lnl = log(nlast);
  double mx = -INFINITY;
  for (int J = threadIdx.x; J < n; J += kThreads) {
    pout[J] = static_cast<float>(pv[J]);
    const double x = S[J] + spread_gain(s2r[J], J == n - 1 ? lnl : lnf);
    pv[J] = x;
    mx = fmax(mx, x);
  }
  mx = block_max_d(mx, r);
  double sum = 0.0;
  for (int J = threadIdx.x; J < n; J += kThreads) {
    const double e = exp(pv[J] - mx);
    pv[J] = e;
    sum += e;
  }
  sum = block_sum_d(sum, r);
  const double price = a.price, cost_skip = 1.5 / static_cast<double>(dm.Bk);
  const double cu = 2.0 * kE4m3U * kE4m3U / 3.0, dd = static_cast<double>(dm.D) * static_cast<double>(dm.D);
  const double cu4 = 2.0 * kE2m1U * kE2m1U / 3.0;
  const bool skim = a.tau_skim > 0.0f;
  for (int J = threadIdx.x; J < n; J += kThreads) {
    PriceTile x;
    x.s2 = s2r[J];
    x.n = J == n - 1 ? nlast : nfull;
    x.vnorm = vnorm[J];
    x.vvar = vvar[J];
    x.m2v = m2v[J];
    {
#pragma clang fp contract(off)
      x.sl2 = cu * (m2q * static_cast<double>(m2k[J])) / dd;
      x.sk2 = cu4 * (m2q * static_cast<double>(m2k[J])) / dd;
    }
    tr[J] = price_tier(x, pv[J] / sum, price, cost_skip, skim);
  }
}

// K2B_PRICE is the tier pass of the price router: its error model needs many
// more registers, so it is an instance of its own and the other modes keep
// their occupancy.
enum { K2B_TIERS = 0, K2B_ENTROPY = 1, K2B_PRICE = 2 };

inline size_t k2b_lds_bytes(int nk) { return ((size_t)nk * 9 + 15) / 16 * 16; }

// One workgroup per (b, h, I) (tiers) or per (b, h, sampled row s) (entropy).
template <int WHAT>
__global__ __launch_bounds__(kThreads) void k2b_rows(RouterArgs a) {
  // row buffers sized by the launch for this Nk: p (f64), tiers
  extern __shared__ __attribute__((aligned(16))) unsigned char k2b_dyn[];
  __shared__ Red r;
  const Dims& dm = a.d;
  const int n = dm.Nk;
  double* pv = reinterpret_cast<double*>(k2b_dyn);
  unsigned char* tr = k2b_dyn + (size_t)n * 8;
  int bh, I, s = 0;
  if (WHAT == K2B_ENTROPY) {
    const int S = min(a.samples, dm.Nq);
    bh = blockIdx.x / S;
    s = blockIdx.x % S;
    I = (int)(((int64_t)s * dm.Nq) / S);
  } else {
    bh = blockIdx.x / dm.Nq;
    I = blockIdx.x % dm.Nq;
  }
  const int64_t row = (int64_t)bh * dm.Nq + I;
  const double* S = reinterpret_cast<const double*>(a.ws + a.L.S) + row * n;
  if (a.mode != TATTN_MODE_ALL_FULL) {
    double mx = -INFINITY;
    for (int J = threadIdx.x; J < n; J += kThreads) {
      pv[J] = S[J];
      mx = fmax(mx, pv[J]);
    }
    mx = block_max_d(mx, r);
    double sum = 0.0;
    for (int J = threadIdx.x; J < n; J += kThreads) {
      const double e = exp(pv[J] - mx);
      pv[J] = e;
      sum += e;
    }
    sum = block_sum_d(sum, r);
    for (int J = threadIdx.x; J < n; J += kThreads) pv[J] = pv[J] / sum;
    __syncthreads();
  }
  if (WHAT == K2B_ENTROPY) {
    double hsum = 0.0;
    for (int J = threadIdx.x; J < n; J += kThreads) hsum += pv[J] > 0.0 ? pv[J] * log(pv[J]) : 0.0;
    hsum = block_sum_d(hsum, r);
    if (threadIdx.x == 0) reinterpret_cast<double*>(a.ws + a.L.ent)[(int64_t)bh * min(a.samples, dm.Nq) + s] = -hsum;
    return;
  }
  float* pout = reinterpret_cast<float*>(a.ws + a.L.p) + row * n;
  unsigned char* tout = a.ws + a.L.tiers + row * n;
  if constexpr (WHAT == K2B_PRICE) {
    price_row(a, bh, row, S, pv, tr, pout, r);
  } else if (a.mode == TATTN_MODE_ALL_FULL) {
    for (int J = threadIdx.x; J < n; J += kThreads) {
      tr[J] = TATTN_FULL;
      pout[J] = 0.0f;
    }
  } else if (a.mode == TATTN_MODE_THRESHOLD) {
    const double th = a.tau_hi, tl = a.tau_lo, tk = a.tau_skim;
    for (int J = threadIdx.x; J < n; J += kThreads) {
      const double p = pv[J];
      tr[J] = p >= th ? TATTN_FULL : p >= tl ? TATTN_LOW : (tk > 0.0 && p >= tk) ? TATTN_SKIM : TATTN_SKIP;
      pout[J] = static_cast<float>(p);
    }
    if (a.top_k > 0) {
      __syncthreads();
      mark_top_k(pv, n, a.top_k, [&](int J, bool kept) { if (!kept) tr[J] = TATTN_SKIP; }, r);
    }
  } else {  // ADAPTIVE
    const int S2 = min(a.samples, dm.Nq);
    const double* ent = reinterpret_cast<const double*>(a.ws + a.L.ent) + (int64_t)bh * S2;
    // block-parallel sum of the head's sampled entropies: a fixed reduction
    // tree, so every workgroup of this head gets the same k_h
    double hv = 0.0;
    for (int i = threadIdx.x; i < S2; i += kThreads) hv += ent[i];
    const double hs = block_sum_d(hv, r);
    double rr = exp(hs / S2) / n;
    rr = fmin(fmax(rr, (double)a.keep_min), (double)a.keep_max);
    const int kh = (int)ceil(rr * n);
    const int nfull = (int)ceil((double)a.full_frac * kh);
    if (I == 0 && threadIdx.x == 0) {
      reinterpret_cast<int*>(a.ws + a.L.kh)[bh] = kh;
      reinterpret_cast<double*>(a.ws + a.L.rh)[bh] = rr;
    }
    // the FULL cut (rank nfull <= kh) lies at or above the k_h-th largest, so
    // its select only counts the values from there up
    const uint64_t xk = mark_top_k(pv, n, kh, [&](int J, bool kept) { tr[J] = kept ? TATTN_LOW : TATTN_SKIP; }, r);
    mark_top_k(pv, n, nfull, [&](int J, bool kept) { if (kept) tr[J] = TATTN_FULL; }, r, xk);
    if (a.tau_skim > 0.0f) {   // the fourth tier: a tile outside the top k_h with p >= tau_skim
      __syncthreads();
      const double tk = a.tau_skim;
      for (int J = threadIdx.x; J < n; J += kThreads)
        if (tr[J] == TATTN_SKIP && pv[J] >= tk) tr[J] = TATTN_SKIM;
    }
    for (int J = threadIdx.x; J < n; J += kThreads) pout[J] = static_cast<float>(pv[J]);
  }
  __syncthreads();
  int j0, j1;
  diag_range(dm, I, j0, j1);
  for (int J = j0 + threadIdx.x; J <= j1; J += kThreads) tr[J] = TATTN_FULL;
  __syncthreads();
  for (int J = threadIdx.x; J < n; J += kThreads) tout[J] = tr[J];
  compact_row(tr, n, dm.Bk, reinterpret_cast<int16_t*>(a.ws + a.L.lists) + row * n,
              reinterpret_cast<int*>(a.ws + a.L.counts) + row * 4, r);
}

__global__ __launch_bounds__(kThreads) void k2c_compact(RouterArgs a) {
  __shared__ unsigned char tr[kRouterMaxNk];
  __shared__ Red r;
  const Dims& dm = a.d;
  const int n = dm.Nk;
  const int bh = blockIdx.x / dm.Nq, I = blockIdx.x % dm.Nq;
  const int64_t row = (int64_t)bh * dm.Nq + I;
  unsigned char* tg = a.ws + a.L.tiers + row * n;
  for (int J = threadIdx.x; J < n; J += kThreads) tr[J] = tg[J];
  __syncthreads();
  int j0, j1;
  diag_range(dm, I, j0, j1);
  for (int J = j0 + threadIdx.x; J <= j1; J += kThreads) tr[J] = TATTN_FULL;
  __syncthreads();
  for (int J = threadIdx.x; J < n; J += kThreads) tg[J] = tr[J];
  compact_row(tr, n, dm.Bk, reinterpret_cast<int16_t*>(a.ws + a.L.lists) + row * n,
              reinterpret_cast<int*>(a.ws + a.L.counts) + row * 4, r);
}

// ------------------------------------------------------------------ K2d work order
// The fused kernel takes its (b, h, I) work items in the order written here.
// Rows stay in their natural head-major order (a couple of heads in flight, so
// their K/V stay in the shared last-level cache) except the last kTailRows,
// which are sorted by descending step count: the longest rows start first and
// the short ones fill the slots that free up at the end, so the grid does not
// finish on a few long rows.  Rows with equal counts land in any order (the
// result of every row is independent of when it runs).
constexpr int kTailRows = 2048;
constexpr int kOrderThreads = 1024;
constexpr int kOrderBins = 8192;   // step counts: <= Nk + 2 * ceil(Nk / 64) < 8192
constexpr int kBinsPerThread = kOrderBins / kOrderThreads;

__global__ __launch_bounds__(kOrderThreads) void k2d_order(RouterArgs a) {
  __shared__ int hist[kOrderBins];   // indexed by u = kOrderBins - 1 - count (descending counts)
  __shared__ int wsum[kOrderThreads / 64];
  const Dims& dm = a.d;
  const int total = dm.BH * dm.Nq;
  const int T = min(total, kTailRows), head = total - T;
  const int* counts = reinterpret_cast<const int*>(a.ws + a.L.counts);
  int* order = reinterpret_cast<int*>(a.ws + a.L.order);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int i = t; i < head; i += kOrderThreads) order[i] = i;
  for (int i = t; i < kOrderBins; i += kOrderThreads) hist[i] = 0;
  __syncthreads();
  for (int i = t; i < T; i += kOrderThreads)
    atomicAdd(&hist[kOrderBins - 1 - min(counts[(head + i) * 4 + 3], kOrderBins - 1)], 1);
  __syncthreads();
  // exclusive prefix over u: thread t owns u in [8t, 8t + 8)
  int loc[kBinsPerThread], sum = 0;
#pragma unroll
  for (int j = 0; j < kBinsPerThread; j++) {
    loc[j] = hist[kBinsPerThread * t + j];
    sum += loc[j];
  }
  int inc = sum;   // inclusive scan of the thread sums inside the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(inc, o, 64);
    if (lane >= o) inc += up;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int base = 0;
  for (int ww = 0; ww < w; ww++) base += wsum[ww];
  int run = base + inc - sum;
#pragma unroll
  for (int j = 0; j < kBinsPerThread; j++) {
    hist[kBinsPerThread * t + j] = run;
    run += loc[j];
  }
  __syncthreads();
  for (int i = t; i < T; i += kOrderThreads) {
    const int u = kOrderBins - 1 - min(counts[(head + i) * 4 + 3], kOrderBins - 1);
    order[head + atomicAdd(&hist[u], 1)] = head + i;
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  const Dims& d = a.d;
  if (d.Nk > kRouterMaxNk) return hipErrorInvalidValue;
  if (a.mode != TATTN_MODE_ALL_FULL) {
    dim3 grid((d.Nk + 63) / 64, (d.Nq + 63) / 64, d.BH);
    if (d.D == 128)
      hipLaunchKernelGGL((k2a_scores<128, false>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k2a_scores<64, false>), grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.mode == TATTN_MODE_PRICE) {
    dim3 grid((d.Nk + 63) / 64, (d.Nq + 63) / 64, d.BH);
    if (d.D == 128)
      hipLaunchKernelGGL((k2a_scores<128, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k2a_scores<64, true>), grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.mode == TATTN_MODE_ADAPTIVE) {
    const int S = min(a.samples, d.Nq);
    hipLaunchKernelGGL((k2b_rows<K2B_ENTROPY>), dim3(d.BH * S), dim3(kThreads), k2b_lds_bytes(d.Nk), s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.mode == TATTN_MODE_PRICE)
    hipLaunchKernelGGL((k2b_rows<K2B_PRICE>), dim3(d.BH * d.Nq), dim3(kThreads), k2b_lds_bytes(d.Nk), s, a);
  else
    hipLaunchKernelGGL((k2b_rows<K2B_TIERS>), dim3(d.BH * d.Nq), dim3(kThreads), k2b_lds_bytes(d.Nk), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k2d_order, dim3(1), dim3(kOrderThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const RouterArgs& a, hipStream_t s) {
  const Dims& d = a.d;
  if (d.Nk > kRouterMaxNk) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k2c_compact, dim3(d.BH * d.Nq), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k2d_order, dim3(1), dim3(kOrderThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tattn
