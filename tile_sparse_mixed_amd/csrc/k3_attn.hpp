// K3: the fused three-tier attention pass ("Triage": skip / low precision /
// full tiles executed in a single pass; "APT": dual-precision compute units
// and a tile dataflow; "FG-Attn": dense work only on kept tiles).
//
// One workgroup per (b, h, query block I) of BQ = 32 * NW rows; wave w owns
// rows 32w..32w+31 and computes S^T = K Q^T, so each lane holds one query
// column and its softmax statistics stay inside the lane pair (l, l^32).
// The workgroup walks a sequence of 64-key steps:
//   FULL      a kept tile: K and V rows of the caller's bf16 tensors; S^T on
//             v_mfma_f32_32x32x16_bf16, O^T += V^T P^T on the same
//             instruction with P in bf16 and the V^T operand read from the V
//             rows by the transposing LDS read (no V copy in the plan),
//   LOW       a low-precision tile: S^T on v_mfma_f32_32x32x64_f8f6f4 from the
//             E4M3 copies of Q and K scaled by sq*sk; the probabilities
//             quantised to E4M3 against the tile's row maximum (448 at the
//             maximum); O^T += V8^T P8^T on the same fp8 instruction against the
//             E4M3 V, merged with the weight 2^(tile max - m) * sv / 448, and
//             the row sum of the codes from one more fp8 MFMA against ones
//             (blocks below 64 keys: the quantised probabilities times their
//             block's weight in fp16, P.V on the fp16 MFMA against the fp16
//             dequantised V, since one fp8 P.V there would mix blocks of
//             different scales),
//   SKIP_S    64 pooled keys kbar_J of one chunk of 64 key blocks, as a bf16
//             hi + lo pair (two MFMAs: ~2^-17 precision), each scored with a
//             log2(n_J) bias if J is skipped in this row and -inf otherwise
//             ("Triage": a skipped tile is one score weighted by n_J),
//   SKIP_PV   the same chunk's block means vbar_J (fp16, transposed) for P.V,
//   SKIM      (instances with SKIM = true, 64-key blocks) a 4-bit tile: S^T on
//             the same instruction with MXFP4 operands and their E8M0 block
//             scales ("Triage": skimming in 4 bits); probabilities and P.V as
//             in LOW.
// Skipped blocks are visited as whole chunks of 64 (contiguous operands),
// masked to the row's SKIP set; chunks with no skipped block are not visited.
// With 16-key blocks ("FG-Attn": M x N tiles with a small N, down to N = 1)
// a FULL or LOW step gathers up to four consecutive entries of the row's list
// into one 64-key step; with blocks of BK <= 8 keys it gathers 64 / BK (slots,
// down to one key each).  The K, V, E4M3 K and low-tier V rows of a block go
// to score rows chosen so that its keys are consecutive P values of one lane
// half (slotg / kkg); the V^T operand is read from the V rows by the
// transposing LDS read, so any placement of keys on score rows works.
//
// Data movement: every step's operands go global -> LDS with direct
// buffer_load_dwordx4 ... lds (no staging registers) into one of two stage
// buffers while the other stage is computed.  The two stages are distinct
// __shared__ arrays and every step knows its stage at compile time (the step
// loops are unrolled by two): the compiler's wait insertion then sees that the
// DMA into one stage cannot alias the operand reads of the other and does not
// put a vmcnt(0) in front of them, which would serialise the copy and the
// math.  Two-wave workgroups keep one stage instead, as two arrays for its
// halves, and refill each half as soon as its reads are done (see SPLIT).
// Scalar buffer resources carry
// the bases, so a lane needs one 32-bit offset per load pattern, and a
// per-tile resource over the caller's K returns zeros for rows past N.  The
// XOR swizzle that keeps the MFMA operand reads bank-conflict free is applied
// by choosing each lane's source offset.  A step ends with vmcnt(0) +
// s_barrier, which publishes the next stage; the plain barrier (no fence)
// keeps the next step's DMA in flight during the current step's math.
//
// Running state per lane: m (base-2 reference), l (sum of the weights
// relative to 2^m) and the O^T accumulator.  m is raised only when a tile's
// max exceeds it by more than 8, so most steps skip the rescale.
//
// The LOW-tier Q scales are taken here from the Q block the kernel is given
// (its amax over the workgroup), so a forward with other queries than the
// plan's keeps the low tier exact to its definition.  Instances with DUMP =
// true also write every LOW and SKIM step's probability codes of the rows the
// caller selected (tattn_forward_dump).
#pragma once

#include <type_traits>

#include "tattn_device.hpp"
#include "tattn_internal.hpp"

// Every fused multiply-add below is written out; no other product is fused
// with a sum, so every instance of the kernel (with or without the code dump)
// rounds the same operations the same way.
#pragma clang fp contract(off)

namespace tattn {
namespace {

constexpr float kLazy = 8.0f;   // raise m only when a tile max exceeds it by this much (log2)

enum StepKind { kFull = 0, kLow = 1, kSkipS = 2, kSkipPV = 3, kSkim = 4 };

typedef __attribute__((address_space(3))) void lds_void;

// vmcnt(0) with expcnt and lgkmcnt unconstrained (gfx9 s_waitcnt encoding).
__device__ inline void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// vmcnt(0) and lgkmcnt(0): this wave's DMA has landed and its LDS reads have
// returned (the compiler may leave the last operand reads of a step in flight
// and consume them after the barrier, while other waves already refill that
// stage).
__device__ inline void wait_vm0_lgkm0() { __builtin_amdgcn_s_waitcnt(0x0070); }

// lgkmcnt(0) alone: this wave's LDS reads (and scalar loads) have returned.
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// vmcnt(n): at most this wave's n newest vector-memory instructions still in
// flight (they complete in issue order).  n is wave-uniform; past 8 it waits
// for all, which is only slower.
__device__ inline void wait_vm_n(int n) {
  switch (n) {
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

// One wave: copy 64 lanes x 16 bytes into LDS[dst .. dst+1024); lane l's bytes
// come from byte offset voff (per lane) + soff (uniform) of buffer `r`.  A
// read past the buffer's num_records returns zeros.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
}

// max(x of lane l, x of lane l ^ 32): v_permlane32_swap exchanges the two
// halves of the wave between two registers without an LDS round trip
__device__ inline float max_lane_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Pins the schedule of a run of n (LDS read, MFMA) pairs: `ahead` reads are
// issued first, then each MFMA is followed by the next read, so `ahead` reads
// stay in flight instead of each MFMA waiting on a just-issued read.
template <int N, int AHEAD>
__device__ inline void pipeline_reads_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);   // DS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// The same for operands of two LDS reads each (the transposing V reads):
// `ahead` operands' reads first, then each MFMA followed by the next
// operand's two reads.
template <int N, int AHEAD>
__device__ inline void pipeline_reads2_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);   // DS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);         // DS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Schedule of one software-pipelined low-tier step (one basic block): the
// next step's K reads, its D/32 score MFMAs spread through this step's
// softmax VALU, the row-sum MFMA, the V reads, then each P.V MFMA behind the
// 16 multiplies of the accumulator block it consumes.
template <int D>
__device__ inline void schedule_low_step() {
  __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);     // DS reads: next step's K codes
#pragma unroll
  for (int i = 0; i < D / 32; i++) {
    __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);       // VALU: this step's softmax
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA: next step's scores
  }
  __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA: row sum of the codes
  __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);     // DS reads: this step's V codes
#pragma unroll
  for (int i = 0; i < D / 32; i++) {
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);       // VALU: accumulator block i times wr
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA: P.V into block i
  }
}

// Schedule of a pipelined refined low-tier step: per score block of the next
// step its K4, residual and scale-word reads, then its 3 D/64 fp4 MFMAs
// spread through this step's quantisation; the row-sum MFMA; then the P.V as
// in schedule_low_step.
template <int D>
__device__ inline void schedule_refine_step() {
#pragma unroll
  for (int b = 0; b < 2; b++) {
    __builtin_amdgcn_sched_group_barrier(0x100, D / 32 + 2, 0);   // DS reads: one score block's K operands
#pragma unroll
    for (int i = 0; i < 3 * D / 64; i++) {
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);          // VALU: this step's quantisation
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA: next step's scores
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA: row sum of the codes
  __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);     // DS reads: this step's V codes
#pragma unroll
  for (int i = 0; i < D / 32; i++) {
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);       // VALU: accumulator block i times wr
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA: P.V into block i
  }
}

// LDS swizzles.  An MFMA operand read has the lanes of a half-wave read 16
// bytes at the same logical chunk of 32 consecutive rows.  gfx950 serves a
// ds_read_b128 16 lanes at a time across 64 four-byte banks (256 bytes), so
// 16 consecutive rows must land on 16 distinct 16-byte slots modulo 256; the
// chunk index is XORed with a function of the row chosen so that this holds
// (and also 8 rows modulo 128 bytes).  Measured: XORing with (row & 7) alone
// left ~1 bank-conflict cycle per LDS access.
__device__ inline int swz256(int r) { return r & 15; }                          // 256-byte rows
__device__ inline int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }        // 128-byte rows
__device__ inline int swz64(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }  // 64-byte rows
// Swizzled byte offsets of 16-byte chunk `ch` of a row inside a stage region.
template <int D>
__device__ inline int offK(int row, int ch) {                                   // [64][D] bf16
  return D == 128 ? row * 256 + ((ch ^ swz256(row)) << 4) : row * 128 + ((ch ^ swz128(row)) << 4);
}
__device__ inline int offV(int d, int ch) { return d * 128 + ((ch ^ swz128(d)) << 4); }   // [D][64] 16-bit
// V rows [64][D] 16-bit (FULL tiles): chunk c of row r sits at slot c ^ swzv(r).
// Their P.V operand is read with the transposing LDS read, whose half-wave
// takes four consecutive rows 4u..4u+3 at four chunks each; XORing chunk bit
// 2 (and bit 3 at 256-byte rows) with the row's place in its group of four
// puts those 16 chunks on 16 distinct slots modulo 256 bytes.
template <int D>
__device__ inline int swzv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
template <int D>
__device__ inline int offK8(int row, int ch) {                                  // [64][D] bytes
  return D == 128 ? row * 128 + ((ch ^ swz128(row)) << 4) : row * 64 + ((ch ^ swz64(row)) << 4);
}

// score scale of a staged step: one value for 64-key blocks, one per 16-key
// group for 16-key blocks; with blocks of <= 8 keys the factor common to the
// step (sq * log2(e) / sqrt(d) on LOW steps) and, per lane g < G, the E4M3 K
// scale of slot g (read per lane by the step's P values)
template <int G>
struct StepScale {
  static constexpr int N = G == 4 ? 4 : 1;
  float c[N];
  float kv;  // blocks of <= 8 keys, LOW steps: lane g < G holds slot g's sk
  float v;   // E4M3 value scale of a 64-key LOW or SKIM step's block
};

// SKIM: the instance also runs the SKIM tier; the other instances carry none
// of its code.  DUMP: the probability-code dump.
// REFINE: LOW tiles score on MXFP4 copies of Q and K with an MXFP4 residual
// correction, <q4,k4> + <q4,k4r> + <q4r,k4> on the block-scaled fp4 MFMA
// ("Triage": refining a tile with 4-bit residual correction); their
// probabilities and P.V are the low tier's.  R0 of such a step holds K4 rows
// [64][D/2] at 0, their scale words at 32 D, the residual rows at 64 D and
// their scale words at 96 D (gathered per slot with blocks below 64 keys).
template <int D, int NW, int BK, bool SKIM, bool DUMP, bool REFINE>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2)))
void k3_attn(AttnArgs a) {
  static_assert(BK == 64 || BK == 16 || BK == 8 || BK == 4 || BK == 2 || BK == 1,
                "key blocks are 64, 16, 8, 4, 2 or 1 keys");
  static_assert(!REFINE || !SKIM, "the refined low tier runs without the SKIM tier");
  constexpr int G = 64 / BK;          // key blocks per 64-key step
  constexpr int R1 = 128 * D;         // bytes of each half of a stage (R0: K-side operands, R1: V-side)
  // Two-wave workgroups (64-row query blocks) keep ONE stage and refill its
  // halves in turn: the K half of step t+1 while step t runs its softmax and
  // P.V, the V half while step t+1 scores.  That halves their LDS, so a CU
  // holds four of them (two waves per SIMD) instead of two (one per SIMD).
  // The halves are then two arrays (stA = R0, stB = R1), so that the
  // compiler's wait insertion sees a DMA into one half never alias reads of
  // the other.
  constexpr bool SPLIT = NW == 2;
  // Four-wave workgroups keep two stages, each as two arrays (R0 and R1):
  // the software-pipelined low phase refills the R0 half of one stage while
  // the R1 half of the same stage is read, and separate arrays let the wait
  // insertion see that these never alias.
  __shared__ __attribute__((aligned(1024))) unsigned char stA[R1];   // R0 of even steps (two-wave: the one stage's R0)
  __shared__ __attribute__((aligned(1024))) unsigned char stB[R1];   // R0 of odd steps (two-wave: the one stage's R1)
  __shared__ __attribute__((aligned(1024))) unsigned char svA[SPLIT ? 16 : R1];   // R1 of even steps
  __shared__ __attribute__((aligned(1024))) unsigned char svB[SPLIT ? 16 : R1];   // R1 of odd steps
  // the R1 region of a stage
  auto r1 = [&](const unsigned char* st) __attribute__((always_inline)) -> unsigned char* {
    if constexpr (SPLIT) return stB;
    else return st == stA ? svA : svB;
  };
  extern __shared__ int16_t slist[];         // the row's FULL, LOW (and SKIM) key blocks (list_cap entries)
  __shared__ uint64_t smask[64];             // per visited chunk: bit j = block 64c + j skipped
  __shared__ unsigned char schunk[64];       // chunks holding at least one skipped block
  __shared__ int snc;
  __shared__ float samax[NW];                // per wave: max |q| of its rows

  const Dims& dm = a.d;
  // ---- work mapping: workgroup x takes row (b, h, I) = order[x], which is the
  // row-major order except that the last rows are sorted longest first (the
  // router's work order).  The dispatcher deals consecutive workgroups
  // round-robin to the 8 XCDs, so the ~2 heads in flight at a time are shared
  // by all XCDs and their K/V tiles (~34 MB per head at d = 128) stay resident
  // in the shared 256 MB MALL.  Giving each XCD its own contiguous range of
  // heads instead put 8 heads in flight (~270 MB) and measured ~15x the
  // compulsory HBM reads.
  const int w_item = reinterpret_cast<const int*>(a.ws + a.L.order)[blockIdx.x];
  const int bh = w_item / dm.Nq, I = w_item % dm.Nq;
  const int bidx = bh / dm.H, hidx = bh % dm.H;
  const int64_t toff = (int64_t)bidx * dm.sb + (int64_t)hidx * dm.sh;
  const int64_t row = (int64_t)bh * dm.Nq + I;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, lh = lane >> 5;

  // ---- Q rows of this wave as bf16 B operands: lane (ln, lh) holds
  // q[row][16c + 8lh .. +8] for chunk c; rows past N are zero.
  const int qrow = I * (32 * NW) + wave * 32 + ln;
  bf16x8 qreg[D / 16];
  {
    uint32_t mx = 0;   // largest |q| of the lane's values, as bf16 bits (monotone in the magnitude)
#pragma unroll
    for (int c = 0; c < D / 16; c++) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qrow < dm.N) v = *reinterpret_cast<const uint4*>(a.q + toff + (int64_t)qrow * dm.sn + 16 * c + 8 * lh);
      qreg[c] = __builtin_bit_cast(bf16x8, v);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; j++) mx = max(mx, max(w4[j] & 0x7fffu, (w4[j] >> 16) & 0x7fffu));
    }
    const float am = wave_max(__uint_as_float(mx << 16));
    if (lane == 0) samax[wave] = am;
  }

  const unsigned char* ws = a.ws;
  const int* counts = reinterpret_cast<const int*>(ws + a.L.counts) + row * 4;
  // the list in LDS holds a.list_cap entries, the plan's bound on a row's kept
  // tiles; a row past it (not possible for a valid plan) is cut, never read past
  const int cap = a.list_cap;
  const int nF = min(counts[0], cap), nL = min(counts[1], cap - nF);
  const int nK = nF + nL;
  const int nSk = SKIM ? min(dm.Nk - counts[0] - counts[1] - counts[2], cap - nK) : 0;   // SKIM follows LOW
  if (tid == 0 && counts[0] + counts[1] + (SKIM ? dm.Nk - counts[0] - counts[1] - counts[2] : 0) > cap)
    atomicOr(reinterpret_cast<int*>(a.ws + a.L.flag), 1);   // reported by tattn_plan_stats
  {
    const int16_t* list = reinterpret_cast<const int16_t*>(ws + a.L.lists) + row * dm.Nk;
    for (int i = tid; i < nK + nSk; i += NW * 64) slist[i] = list[i];
  }
  if (wave == 0) {   // lane c: the skip mask of key-block chunk c, from the tier row
    const unsigned char* tiers = ws + a.L.tiers + row * dm.Nk;
    uint64_t m = 0;
    if (lane < dm.NkC) {
      const int j0 = 64 * lane, n = min(64, dm.Nk - j0);
      for (int j = 0; j < n; j++) m |= static_cast<uint64_t>(tiers[j0 + j] == TATTN_SKIP) << j;
    }
    const bool has = m != 0;
    const uint64_t bal = __ballot(has);
    if (has) {
      const int ci = __popcll(bal & ((1ull << lane) - 1));
      schunk[ci] = static_cast<unsigned char>(lane);
      smask[ci] = m;
    }
    if (lane == 0) snc = __popcll(bal);
  }
  __syncthreads();
  const int sF = (nF + G - 1) / G, sL = (nL + G - 1) / G;   // FULL / LOW steps
  const int sSk = (nSk + G - 1) / G;                         // SKIM steps
  const int nSteps = sF + 2 * snc + sL + sSk;

  const uint16_t* kin = a.k + toff;
  const uint16_t* vin = a.v + toff;
  const unsigned char* slab = ws + a.L.slab + (int64_t)bh * a.L.sl.bytes;
  const Slab SL = a.L.sl;
  // sk is read through the constant address space: a uniform load there is a
  // scalar load, counted by lgkmcnt, so waiting for it does not also wait for
  // the DMA already in flight (a vector load would share vmcnt with it).
  typedef __attribute__((address_space(4))) const float cfloat;
  cfloat* skp = (cfloat*)(reinterpret_cast<const float*>(ws + a.L.sk) + (int64_t)bh * dm.Nk);
  cfloat* svp = (cfloat*)(reinterpret_cast<const float*>(ws + a.L.sv) + (int64_t)bh * dm.Nk);
  const float* skg = reinterpret_cast<const float*>(ws + a.L.sk) + (int64_t)bh * dm.Nk;   // per-lane loads

  const float cF = kLog2e / __builtin_sqrtf(static_cast<float>(D));
  // the Q block's E4M3 scale and its inverse, from the block's amax (as the
  // pooling kernel forms them: a float64 quotient rounded once)
  float sq, iq;
  {
    float am = samax[0];
#pragma unroll
    for (int w = 1; w < NW; w++) am = __builtin_fmaxf(am, samax[w]);
    sq = am == 0.0f ? 1.0f : static_cast<float>(static_cast<double>(am) / 448.0);
    iq = am == 0.0f ? 1.0f : static_cast<float>(448.0 / static_cast<double>(am));
  }

  // step order: the skip chunks (score / P.V pairs), then FULL tiles, then LOW
  // tiles, so the bf16 Q registers are dead before the E4M3 copy is made, then
  // SKIM tiles.  (Skip chunks first: their loop then starts at an even step
  // and is generated once, not once per stage parity, and the kernel fits its
  // registers without spilling; with FULL first it spilled 42 VGPRs whose
  // scratch reloads share vmcnt with the DMA.)
  const int nS2 = 2 * snc, tLow = nS2 + sF, tSk = tLow + sL;
  auto step_kind = [&](int t) __attribute__((always_inline)) {
    if (t < nS2) return (t & 1) ? (int)kSkipPV : (int)kSkipS;
    if (t < tLow) return (int)kFull;
    if (SKIM && t >= tSk) return (int)kSkim;
    return (int)kLow;
  };
  // list entry of key block g of a FULL, LOW or SKIM step, and the end of its list
  auto list_idx = [&](int t, int g) {
    return t < tLow ? G * (t - nS2) + g : (SKIM && t >= tSk) ? nK + G * (t - tSk) + g : nF + G * (t - tLow) + g;
  };
  auto list_end = [&](int t) { return t < tLow ? nF : (SKIM && t >= tSk) ? nK + nSk : nK; };
  auto list_at = [&](int t) { return (int)slist[list_idx(t, 0)]; };

  // ---- DMA of step t's operands into stage `st`.  Region layouts (bytes):
  //   FULL    R0 = K [64][D] bf16,       R1 = V [64][D] bf16 (the caller's rows)
  //   LOW     R0 = K8 [64][D] E4M3,      R1 = V8^T [D][64] E4M3 (64-key blocks)
  //                                         or V low [64][D] fp16 rows (16, 8)
  //   SKIM    R0 = K4 [64][D/2] + scales, R1 = V8^T [D][64] E4M3
  //   SKIP_S  R0 = kbar hi [64][D] bf16, R1 = kbar lo [64][D] bf16
  //   SKIP_PV                            R1 = vbar^T [D][64] fp16
  // Wave w issues the 1 KB instructions k = w, w + NW, ...  A 16-bit row of D
  // elements spans D/8 chunks, so one instruction covers RPI = 1024/(2D) rows.
  constexpr int CH = D / 8, RPI = 1024 / (2 * D), NI16 = D / 8 / NW, NI8 = D / 16 / NW;
  const int rr16 = lane / CH, pos16 = lane % CH;   // row within an instruction, chunk slot
  // Per-lane source offsets of a 16-bit [64][D] row tile.  Instruction
  // k = wave + NW i covers rows k RPI .. k RPI + RPI - 1; LDS slot pos16 of row
  // r holds logical chunk pos16 ^ swz(r).  For D = 128, swz256(4k + rr16) =
  // 4 (k & 3) + rr16 takes 4 / NW values over i (NW = 4: one, NW = 2: two, by
  // i & 1); for D = 64, swz128(8k + rr16) = rr16 ^ (k & 1) with k & 1 = wave & 1.
  // So a lane needs NSW offsets, instruction i using index i % NSW.
  constexpr int NSW = D == 128 ? 4 / NW : 1;
  int lk[NSW], lkb[NSW];   // caller's K (row stride sn), pooled K (row stride 2D)
#pragma unroll
  for (int j = 0; j < NSW; j++) {
    const int r = (wave + NW * j) * RPI + rr16;
    const int sw = (pos16 ^ (D == 128 ? swz256(r) : swz128(r))) * 16;
    lk[j] = rr16 * (int)dm.sn * 2 + sw;
    lkb[j] = rr16 * 2 * D + sw;
  }
  // Caller's V rows: instruction k covers rows k RPI + rr16 and RPI is a
  // multiple of 4, so swzv(row) = swzv(rr16) for every instruction.  Formed
  // at each use from an opaque lane index (not held across the loop).
  // rowb: bytes between source rows.
  auto lv_of = [&](int rowb) __attribute__((always_inline)) {
    int lr = lane_here();
    const int r = lr / CH, c = lr % CH;
    return r * rowb + ((c ^ swzv<D>(r)) << 4);
  };
  // [D][64] 16-bit tiles: instruction k covers rows 8k..8k+7, so swz128(r) =
  // ((lane >> 3) & 7) ^ (k & 1), and k & 1 == wave & 1 because NW is even.
  int voffV = (lane >> 3) * 128 + (((lane & 7) ^ ((lane >> 3) & 7) ^ (wave & 1)) * 16);
  // [64][D] E4M3 tiles: 128-byte rows for D = 128 (as above), 64-byte rows for D = 64
  // (instruction k covers rows 16k..16k+15: swz64(r) = ((lane >> 3) & 3) ^ (lane >> 5)).
  int voffK8 = D == 128 ? voffV
                              : (lane >> 2) * 64 + (((lane & 3) ^ ((lane >> 3) & 3) ^ ((lane >> 5) & 1)) * 16);
  // [64][D/2] MXFP4 K tiles (SKIM): an instruction covers 2048/D rows of D/32
  // chunks; LDS slot c of row r holds chunk c ^ swz4(r), swz4(r) = (r >> 2) & 3
  // for 64-byte rows and (r >> 3) & 1 for 32-byte rows, which inside an
  // instruction is (lane >> 4) masked to the chunk count
  constexpr int C4 = D / 32;   // 16-byte chunks per MXFP4 row = scale bytes per row
  const int voffK4 = (lane / C4) * (D / 2) + (((lane & (C4 - 1)) ^ ((lane >> 4) & (C4 - 1))) * 16);
  // [D][64] E4M3 V^T tiles (64-key blocks): 64-byte rows, an instruction covers
  // rows 16k..16k+15; LDS slot c of row r holds chunk c ^ swzv8(r), swzv8(r) =
  // (r >> 2) & 3, which inside an instruction is (lane >> 4) & 3
  const int voffV8 = (lane >> 2) * 64 + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  // one resource over this head's slab; every workspace operand is a scalar
  // sub-offset of it
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(slab, (uint32_t)SL.bytes);
  // 16-key blocks: LDS slot (row d, chunk lane & 7) of a [D][64] 16-bit tile
  // holds logical chunk lc = (lane & 7) ^ swz128(d), i.e. 8 keys of column
  // group lc / 2; the lane fetches them from that group's block, stored
  // [D][16] (32 bytes per row d), half lc & 1 of the row.
  // caller's K and V as one resource per head each for 16- and 8-key gathers:
  // rows past N read as zero
  const __amdgpu_buffer_rsrc_t rKh = make_rsrc(kin, (uint32_t)dm.N * (uint32_t)dm.sn * 2);
  const __amdgpu_buffer_rsrc_t rVh = make_rsrc(vin, (uint32_t)dm.N * (uint32_t)dm.sn * 2);
  // 16-bit rows [64][D] of the step's G blocks from the per-head resource r
  // (the caller's K or V, rows past N reading as zero, or the low tier's V
  // rows), rowb bytes apart, lane offsets off(i) of instruction i.  Score row
  // m holds key m & 15 of block m >> 4 (16-key blocks) or key kkg(m) of slot
  // slotg(m) (blocks of <= 8 keys).
  // jv: lane g < G holds the step's block of slot g
  auto gather16 = [&](__amdgpu_buffer_rsrc_t r, unsigned char* reg, int jv, int rowb, auto off) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI16; i++) {
      const int k = wave + NW * i;
      const int row0 = k * RPI;                // first stage row of the instruction
      if constexpr (G == 4) {
        const int Jg = __builtin_amdgcn_readlane(jv, row0 >> 4);
        dma16(r, reg + k * 1024, off(i) + (Jg * 16 + (row0 & 15)) * rowb, 0);
      } else if constexpr (D == 128 && BK >= 4) {
        // an instruction's four rows are four consecutive keys of one slot
        const int Js = __builtin_amdgcn_readlane(jv, slotg<BK>(row0));
        dma16(r, reg + k * 1024, off(i) + (Js * BK + kkg<BK>(row0)) * rowb, 0);
      } else {
        int lr = lane_here();   // opaque, as for the E4M3 rows below
        const int r16 = lr / CH;
        const int m = row0 + r16;
        dma16(r, reg + k * 1024, off(i) + (__shfl(jv, slotg<BK>(m), 64) * BK + kkg<BK>(m) - r16) * rowb, 0);
      }
    }
  };
  auto load_vt16 = [&](unsigned char* reg, __amdgpu_buffer_rsrc_t r, int base) {   // [D][64] 16-bit
#pragma unroll
    for (int i = 0; i < NI16; i++) {
      const int k = wave + NW * i;
      dma16(r, reg + k * 1024, voffV, base + k * 1024);
    }
  };
  auto load_v8 = [&](unsigned char* reg, int J) __attribute__((always_inline)) {   // [D][64] E4M3 V^T of block J
#pragma unroll
    for (int i = 0; i < NI8; i++) {
      const int k = wave + NW * i;
      dma16(rS, reg + k * 1024, voffV8, (int)SL.v8t + J * 64 * D + k * 1024);
    }
  };
  // MXFP4 K rows of block J and of its residual, with their scale words, into
  // the R0 region `st` of a refined LOW step
  auto refine_k = [&](int J, unsigned char* st) __attribute__((always_inline)) {
    for (int k = wave; k < D / 32; k += NW) {
      dma16(rS, st + k * 1024, voffK4, (int)SL.k4 + J * 32 * D + k * 1024);
      dma16(rS, st + 64 * D + k * 1024, voffK4, (int)SL.k4r + J * 32 * D + k * 1024);
    }
    if (wave == 0 || wave == NW - 1) {
      unsigned char* dst = st + (wave == 0 ? 32 * D : 96 * D);
      const int src = (wave == 0 ? (int)SL.k4s : (int)SL.k4rs) + J * 2 * D;
      if constexpr (D == 128)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)dst, 4, lane * 4, src, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)dst, 2, lane * 2, src, 0, 0);
    }
  };
  // KINDS: bit mask of the step kinds that can occur where this is called; the
  // other branches are not generated, so their address terms are not kept live.
  // PART: 1 = the R0 half (K, E4M3 K, MXFP4 K and its scales, kbar hi) and
  // the step's scales; 2 = the R1 half (V^T, E4M3 V^T or the fp16 low-tier V^T,
  // kbar lo, vbar^T); 3 = both.
  auto issue_part = [&](auto kinds, auto part, int t, unsigned char* st, StepScale<G>& cst) __attribute__((always_inline)) {
    constexpr int KINDS = decltype(kinds)::value;
    constexpr bool PA = decltype(part)::value & 1, PB = decltype(part)::value & 2;
    const int kind = step_kind(t);
    if constexpr (G > 1) {
      if (((KINDS & (1 << kFull)) && kind == kFull) || ((KINDS & (1 << kLow)) && kind == kLow) ||
          (SKIM && (KINDS & (1 << kSkim)) && kind == kSkim)) {
        // one block index per lane (lane g < G: the step's g-th block), read
        // straight from the list; a runtime slot then selects by lane, never by
        // indexing an array (which the compiler would place in scratch memory)
        int jv;
        {
          const int i0 = list_idx(t, 0), e = list_end(t), g = lane & (G - 1);
          jv = (int)slist[i0 + g < e ? i0 + g : i0];
        }
        if ((KINDS & (1 << kFull)) && kind == kFull) {
          if constexpr (PA) gather16(rKh, st, jv, (int)dm.sn * 2, [&](int i) { return lk[i % NSW]; });
          if constexpr (PB) {
            const int lv = lv_of((int)dm.sn * 2);
            gather16(rVh, r1(st), jv, (int)dm.sn * 2, [&](int) { return lv; });
          }
          if constexpr (PA) {
#pragma unroll
            for (int g = 0; g < StepScale<G>::N; g++) cst.c[g] = cF;
          }
        } else if (SKIM && (KINDS & (1 << kSkim)) && kind == kSkim) {
          // MXFP4 K rows (D/2 bytes) per lane from their slots, then one
          // scale word per row (wave 0; a 4-byte LDS slot per lane)
          if constexpr (PA) {
            int lr = lane_here();   // opaque, as for the E4M3 rows below
            constexpr int C4R = D / 32;                  // 16-byte chunks per MXFP4 row
            const int ri = lr / C4R;                     // row of the lane inside an instruction
            // D/32 instructions over NW waves (at d = 64 with four waves, two
            // of them issue none)
#pragma unroll
            for (int i = 0; i < (D / 32 + NW - 1) / NW; i++) {
              const int k = wave + NW * i;
              if constexpr ((D / 32) % NW != 0) {
                if (k >= D / 32) break;
              }
              const int m = k * (2048 / D) + ri;
              const int key = G == 4 ? __shfl(jv, m >> 4, 64) * 16 + (m & 15)
                                     : __shfl(jv, slotg<BK>(m), 64) * BK + kkg<BK>(m);
              dma16(rS, st + k * 1024, (((lr & (C4R - 1)) ^ ((lr >> 4) & (C4R - 1))) << 4) + key * (D / 2), (int)SL.k4);
            }
            if (wave == 0) {
              const int key = G == 4 ? __shfl(jv, lr >> 4, 64) * 16 + (lr & 15)
                                     : __shfl(jv, slotg<BK>(lr), 64) * BK + kkg<BK>(lr);
              if constexpr (D == 128)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(st + 32 * D), 4, key * 4, (int)SL.k4s, 0, 0);
              else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(st + 32 * D), 2, key * 2, (int)SL.k4s, 0, 0);
            }
          }
          if constexpr (PB) {   // the low tier's fp16 V rows, as for LOW steps
            const int lv = lv_of(2 * D) + (int)SL.vlow;
            gather16(rS, r1(st), jv, 2 * D, [&](int) { return lv; });
          }
          if constexpr (PA) {   // the fp4 scores carry their scales: the step's factor only
#pragma unroll
            for (int g = 0; g < StepScale<G>::N; g++) cst.c[g] = cF;
            if constexpr (G >= 8) cst.kv = 1.0f;
          }
        } else if (REFINE && (KINDS & (1 << kLow))) {
          // refined LOW steps: the MXFP4 K rows and their scale words, then the
          // residual's rows and scale words (R0 at 0, 32 D, 64 D, 96 D), per
          // lane from their slots
          if constexpr (PA) {
            const int lr = lane_here();
            constexpr int C4R = D / 32;                  // 16-byte chunks per MXFP4 row
            const int ri = lr / C4R;                     // row of the lane inside an instruction
            const int sw = (((lr & (C4R - 1)) ^ ((lr >> 4) & (C4R - 1))) << 4);
#pragma unroll
            for (int i = 0; i < (D / 32 + NW - 1) / NW; i++) {
              const int k = wave + NW * i;
              if constexpr ((D / 32) % NW != 0) {
                if (k >= D / 32) break;
              }
              const int m = k * (2048 / D) + ri;
              const int key = G == 4 ? __shfl(jv, m >> 4, 64) * 16 + (m & 15)
                                     : __shfl(jv, slotg<BK>(m), 64) * BK + kkg<BK>(m);
              dma16(rS, st + k * 1024, sw + key * (D / 2), (int)SL.k4);
              dma16(rS, st + 64 * D + k * 1024, sw + key * (D / 2), (int)SL.k4r);
            }
            if (wave == 0 || wave == NW - 1) {
              const int key = G == 4 ? __shfl(jv, lr >> 4, 64) * 16 + (lr & 15)
                                     : __shfl(jv, slotg<BK>(lr), 64) * BK + kkg<BK>(lr);
              unsigned char* dst = st + (wave == 0 ? 32 * D : 96 * D);
              const int src = wave == 0 ? (int)SL.k4s : (int)SL.k4rs;
              if constexpr (D == 128)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)dst, 4, key * 4, src, 0, 0);
              else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)dst, 2, key * 2, src, 0, 0);
            }
          }
          if constexpr (PB) {   // the low tier's fp16 V rows
            const int lv = lv_of(2 * D) + (int)SL.vlow;
            gather16(rS, r1(st), jv, 2 * D, [&](int) { return lv; });
          }
          if constexpr (PA) {   // the fp4 scores carry their scales: the step's factor only
#pragma unroll
            for (int g = 0; g < StepScale<G>::N; g++) cst.c[g] = cF;
            if constexpr (G >= 8) cst.kv = 1.0f;
          }
        } else if (KINDS & (1 << kLow)) {
          if constexpr (PA) {
#pragma unroll
            for (int i = 0; i < NI8; i++) {
              const int k = wave + NW * i;
              const int row0 = k * (1024 / D);         // E4M3 rows are D bytes
              if constexpr (G == 4) {
                const int Jg = __builtin_amdgcn_readlane(jv, row0 >> 4);
                dma16(rS, st + k * 1024, voffK8, (int)SL.k8 + (Jg * 16 + (row0 & 15)) * D);
              } else {
                // the lane's terms are recomputed at every step from an opaque
                // lane index: hoisted out of the loop, the per-instruction
                // addresses stayed live across the kernel and spilled
                int lr = lane_here();
                const int ri = D == 128 ? lr >> 3 : lr >> 2;   // row of the lane inside the instruction
                const int m = row0 + ri;
                dma16(rS, st + k * 1024, voffK8 + (__shfl(jv, slotg<BK>(m), 64) * BK + kkg<BK>(m) - ri) * D,
                      (int)SL.k8);
              }
            }
          }
          if constexpr (PB) {   // the low tier's fp16 V rows (slab rows of 2D bytes)
            const int lv = lv_of(2 * D) + (int)SL.vlow;
            gather16(rS, r1(st), jv, 2 * D, [&](int) { return lv; });
          }
          if constexpr (PA) {
            if constexpr (G == 4) {
#pragma unroll
              for (int g = 0; g < 4; g++) cst.c[g] = sq * skp[__builtin_amdgcn_readlane(jv, g)] * cF;
            } else {
              // one vector load (it lands with the step's DMA)
              cst.c[0] = sq * cF;
              cst.kv = skg[jv];
            }
          }
        }
        return;
      }
    }
    if (G == 1 && (KINDS & (1 << kFull)) && kind == kFull) {
      const int J = list_at(t);
      if constexpr (PA) {
        // one resource per tile: rows past N read as zeros (and are masked)
        const uint32_t rows = (uint32_t)min(64, dm.N - J * 64);
        const __amdgpu_buffer_rsrc_t rK = make_rsrc(kin + (int64_t)J * 64 * dm.sn, rows * (uint32_t)dm.sn * 2);
#pragma unroll
        for (int i = 0; i < NI16; i++) {
          const int k = wave + NW * i;
          // the row offset stays in the lane offset: the range check that zeroes
          // rows past N covers the lane offset, not the scalar one
          dma16(rK, st + k * 1024, lk[i % NSW] + k * RPI * (int)dm.sn * 2, 0);
        }
      }
      if constexpr (PB) {
        const uint32_t rows = (uint32_t)min(64, dm.N - J * 64);
        const __amdgpu_buffer_rsrc_t rV = make_rsrc(vin + (int64_t)J * 64 * dm.sn, rows * (uint32_t)dm.sn * 2);
        const int lv = lv_of((int)dm.sn * 2);
#pragma unroll
        for (int i = 0; i < NI16; i++) {
          const int k = wave + NW * i;
          dma16(rV, r1(st) + k * 1024, lv + k * RPI * (int)dm.sn * 2, 0);
        }
      }
      if constexpr (PA) cst.c[0] = cF;
    } else if (G == 1 && (KINDS & (1 << kLow)) && kind == kLow) {
      const int J = list_at(t);
      if constexpr (PA) {
        if constexpr (REFINE) {
          refine_k(J, st);
        } else {
#pragma unroll
          for (int i = 0; i < NI8; i++) {
            const int k = wave + NW * i;
            dma16(rS, st + k * 1024, voffK8, (int)SL.k8 + J * 64 * D + k * 1024);
          }
        }
      }
      if constexpr (PB) load_v8(r1(st), J);
      if constexpr (PA) {
        cst.c[0] = REFINE ? cF : sq * skp[J] * cF;   // refined: the fp4 scales are inside the MFMA
        cst.v = svp[J];
      }
    } else if (G == 1 && SKIM && (KINDS & (1 << kSkim)) && kind == kSkim) {
      // MXFP4 K [64][D/2] into R0, its scale bytes [64][D/32] after it (one
      // D/32-byte load per lane from wave 0, into a 4-byte LDS slot per
      // lane), the E4M3 V^T into R1
      const int J = list_at(t);
      if constexpr (PA) {
        for (int k = wave; k < D / 32; k += NW) dma16(rS, st + k * 1024, voffK4, (int)SL.k4 + J * 32 * D + k * 1024);
        if (wave == 0) {
          if constexpr (D == 128)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(st + 32 * D), 4, lane * 4, (int)SL.k4s + J * 2 * D, 0, 0);
          else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(st + 32 * D), 2, lane * 2, (int)SL.k4s + J * 2 * D, 0, 0);
        }
      }
      if constexpr (PB) load_v8(r1(st), J);
      if constexpr (PA) {
        cst.c[0] = cF;
        cst.v = svp[J];
      }
    } else {
      const int c = schunk[t >> 1];
      if ((KINDS & (1 << kSkipS)) && kind == kSkipS) {
#pragma unroll
        for (int i = 0; i < NI16; i++) {
          const int k = wave + NW * i;
          if constexpr (PA) dma16(rS, st + k * 1024, lkb[i % NSW], (int)SL.kbhi + c * 128 * D + k * 1024);
          if constexpr (PB && BK > 1)   // (one-key blocks: the lo half is zero)
            dma16(rS, r1(st) + k * 1024, lkb[i % NSW], (int)SL.kblo + c * 128 * D + k * 1024);
        }
      } else if (KINDS & (1 << kSkipPV)) {
        if constexpr (PB) load_vt16(r1(st), rS, (int)SL.vbarT + c * 128 * D);
      }
      if constexpr (PA) {
#pragma unroll
        for (int g = 0; g < StepScale<G>::N; g++) cst.c[g] = 1.0f;
      }
    }
  };
  auto issue = [&](auto kinds, int t, unsigned char* st, StepScale<G>& cst) __attribute__((always_inline)) {
    issue_part(kinds, std::integral_constant<int, 3>{}, t, st, cst);
  };

  // ---- per-lane LDS operand offsets, relative to a stage.  Rows 32b + ln have
  // the swizzle of row ln, so the b = 1 half is a constant offset away.  They
  // are made opaque at every step: that keeps the compiler
  // from hoisting one copy of each address per stage out of the loops and
  // lets it fold the stage base into the ds_read immediate instead.
  constexpr int KROW = D == 128 ? 256 : 128;   // bytes per bf16 K row
  constexpr int K8ROW = D;                     // bytes per E4M3 K row
  int offk[D / 16], offv[4], offk8[D / 32], offv8[2];
#pragma unroll
  for (int c = 0; c < D / 16; c++) offk[c] = offK<D>(ln, 2 * c + lh);
#pragma unroll
  for (int c = 0; c < 4; c++) offv[c] = offV(ln, 2 * c + lh);   // within R1
  // E4M3 V^T rows (64 bytes): chunks 2lh, 2lh + 1 of row ln at slots chunk ^ swzv8(ln)
#pragma unroll
  for (int c = 0; c < 2; c++) offv8[c] = ln * 64 + (((2 * lh + c) ^ ((ln >> 2) & 3)) << 4);
#pragma unroll
  for (int i = 0; i < D / 64; i++) {
    const int ch0 = (D == 128 ? 4 * i : 0) + 2 * lh;
    offk8[2 * i] = offK8<D>(ln, ch0);
    offk8[2 * i + 1] = offK8<D>(ln, ch0 + 1);
  }
  auto refresh = [&]() __attribute__((always_inline)) {
    opaque_arr(offk);
    opaque_arr(offv);
    opaque_arr(offk8);
    opaque_arr(offv8);
    opaque_arr(lk);
    opaque_arr(lkb);
    opaque(voffV, voffK8);
  };

  // ---- online-softmax state
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; db++) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  f16x8 pb[4];       // the P operand: fp16, or the bits of bf16 P (FULL tiles)
  i32x8 p8 = {};     // probability codes of a quantised step (LOW, SKIM)
  // From the first quantised 64-key step on, the accumulator holds O^T / accF
  // (relative to 2^m): a step's weight w = 2^(tile max - m) sv / 448 is split
  // into w = wm 2^wk, wm in [1, 2); the MFMA's per-column E8M0 scale applies
  // 2^wk to the codes, the accumulator is multiplied by accF / wm and the
  // MFMA accumulates into it directly, and accF becomes wm.
  float accF = 1.0f;
  float wr = 1.0f;   // accF / wm of the current quantised step
  int wk = 127;      // its E8M0 scale byte, wk + 127
  const int dsl = DUMP ? a.dslot[row] : -1;
  // sum of the fp16 P values the P.V MFMA multiplies, two per
  // v_dot2_f32_f16 (fp32 accumulation), so numerator and denominator see the
  // same rounding
  auto half_sum = [](const f16x8* p) __attribute__((always_inline)) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    float ps = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int j = 0; j < 4; j++) ps = __builtin_amdgcn_fdot2(h2{p[cc][2 * j], p[cc][2 * j + 1]}, one2, ps, false);
    return ps;
  };

  // the same for bf16 P values (v_dot2_f32_bf16)
  auto bf16_sum = [](const f16x8* p) __attribute__((always_inline)) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float ps = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {
      const bf16x8 q = __builtin_bit_cast(bf16x8, p[cc]);
#pragma unroll
      for (int j = 0; j < 4; j++) ps = __builtin_amdgcn_fdot2_f32_bf16(b2{q[2 * j], q[2 * j + 1]}, one2, ps, false);
    }
    return ps;
  };

  // ---- score blocks S^T = K Q^T of the 64 keys of a step (two 32x32 blocks)
  // All operands of a phase are read from LDS before its MFMAs are issued, so
  // the reads overlap each other instead of each waiting on the previous MFMA.
  auto scores_bf16 = [&](const unsigned char* kt, f32x16* s) __attribute__((always_inline)) {
    bf16x8 ka[D / 8];
#pragma unroll
    for (int cq = 0; cq < D / 16; cq++)
#pragma unroll
      for (int b = 0; b < 2; b++) ka[2 * cq + b] = *reinterpret_cast<const bf16x8*>(kt + offk[cq] + b * 32 * KROW);
#pragma unroll
    for (int cq = 0; cq < D / 16; cq++)
#pragma unroll
      for (int b = 0; b < 2; b++) s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2 * cq + b], qreg[cq], s[b], 0, 0, 0);
    pipeline_reads_mfma<D / 8, D / 16>();
  };
  auto scores_fp8 = [&](const unsigned char* kt, f32x16* s, const i32x8* q8) __attribute__((always_inline)) {
    i32x8 ka[D / 32];
#pragma unroll
    for (int i = 0; i < D / 64; i++) {
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const uint4 lo = *reinterpret_cast<const uint4*>(kt + offk8[2 * i] + b * 32 * K8ROW);
        const uint4 hi = *reinterpret_cast<const uint4*>(kt + offk8[2 * i + 1] + b * 32 * K8ROW);
        ka[2 * i + b] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
#pragma unroll
    for (int i = 0; i < D / 64; i++)
#pragma unroll
      for (int b = 0; b < 2; b++)
        s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[2 * i + b], q8[i], s[b], 0, 0, 0, 0, 0, 0);
  };
  // S^T of a refined LOW step: scores_fp4's operand layout, three passes per
  // instruction: K4 x Q4, the K residual x Q4, K4 x the Q residual.
  auto scores_refine = [&](const unsigned char* st, f32x16* s, const i32x8* q4, const int* q4s, const i32x8* q4r,
                           const int* q4rs) __attribute__((always_inline)) {
    const int lsw = lane_here();   // the row swizzle from the hardware lane index (not held across the kernel)
    const int sw = D == 128 ? (lsw >> 2) & 3 : (lsw >> 3) & 1;
    // one score block (32 keys) at a time, its operands read just before its
    // MFMAs: all of them at once would need 32 more registers than the
    // pipelined step has
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const int r = ln + 32 * b;
      uint32_t word, wordr;
      if constexpr (D == 128) {
        word = *reinterpret_cast<const uint32_t*>(st + 32 * D + 4 * r);
        wordr = *reinterpret_cast<const uint32_t*>(st + 96 * D + 4 * r);
      } else {
        word = *reinterpret_cast<const uint16_t*>(st + 32 * D + 4 * r);
        wordr = *reinterpret_cast<const uint16_t*>(st + 96 * D + 4 * r);
      }
      const int ks = static_cast<int>(word >> (8 * lh)), krs = static_cast<int>(wordr >> (8 * lh));
      i32x8 ka[D / 64], kr[D / 64];
#pragma unroll
      for (int i = 0; i < D / 64; i++) {
        const int off = r * (D / 2) + (((2 * i + lh) ^ sw) << 4);
        const uint4 v = *reinterpret_cast<const uint4*>(st + off);
        const uint4 w = *reinterpret_cast<const uint4*>(st + 64 * D + off);
        ka[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        kr[i] = i32x8{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
      }
      // opsel picks byte 2i of the key row's word: the scale of the lane's block
      s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[0], q4[0], s[b], 4, 4, 0, ks, 0, q4s[0]);
      s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr[0], q4[0], s[b], 4, 4, 0, krs, 0, q4s[0]);
      s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[0], q4r[0], s[b], 4, 4, 0, ks, 0, q4rs[0]);
      if constexpr (D == 128) {
        s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[1], q4[1], s[b], 4, 4, 2, ks, 0, q4s[1]);
        s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr[1], q4[1], s[b], 4, 4, 2, krs, 0, q4s[1]);
        s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[1], q4r[1], s[b], 4, 4, 2, ks, 0, q4rs[1]);
      }
    }
  };
  // S^T of a SKIM step on the block-scaled fp4 MFMA: lane (ln, lh) holds
  // channels 64i + 32lh .. +31 of key rows ln and ln + 32 (from the stage) and
  // of its query row (q4, made once per row): one E8M0 block each, whose
  // scale bytes the MFMA applies (opsel picks the byte of the key row's word).
  auto scores_fp4 = [&](const unsigned char* st, f32x16* s, const i32x8* q4, const int* q4s) __attribute__((always_inline)) {
    const int lsw = lane_here();   // the row swizzle from the hardware lane index (not held across the kernel)
    const int sw = D == 128 ? (lsw >> 2) & 3 : (lsw >> 3) & 1;
    if constexpr (SPLIT && G > 1 && D == 128) {
      // one score block at a time (the two-wave instances with gathered
      // steps have no room for both blocks' operands)
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const int r = (lsw & 31) + 32 * b;
        const int ks = static_cast<int>(*reinterpret_cast<const uint32_t*>(st + 32 * D + 4 * r) >> (8 * lh));
        i32x8 kb[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
          const uint4 v = *reinterpret_cast<const uint4*>(st + r * (D / 2) + (((2 * i + lh) ^ sw) << 4));
          kb[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
        s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kb[0], q4[0], s[b], 4, 4, 0, ks, 0, q4s[0]);
        s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kb[1], q4[1], s[b], 4, 4, 2, ks, 0, q4s[1]);
      }
      return;
    }
    i32x8 ka[D / 32];
    int ks[2];
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const int r = ln + 32 * b;
      // the scale DMA gives every lane a 4-byte LDS slot, also for the 2-byte rows of D = 64
      const uint32_t word = D == 128 ? *reinterpret_cast<const uint32_t*>(st + 32 * D + 4 * r)
                                     : static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(st + 32 * D + 4 * r));
      ks[b] = static_cast<int>(word >> (8 * lh));   // byte 2i of ks = scale of block 2i + lh
#pragma unroll
      for (int i = 0; i < D / 64; i++) {
        const uint4 v = *reinterpret_cast<const uint4*>(st + r * (D / 2) + (((2 * i + lh) ^ sw) << 4));
        ka[2 * i + b] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int b = 0; b < 2; b++) {
      s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[b], q4[0], s[b], 4, 4, 0, ks[b], 0, q4s[0]);
      if constexpr (D == 128)
        s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[2 + b], q4[1], s[b], 4, 4, 2, ks[b], 0, q4s[1]);
    }
  };
  // Key of register (b, r) of this lane: 32b + 8(r/4) + 4lh + r%4.  Masks keys
  // >= nvalid (the ragged last tile).
  // Runs once per row; the opaque limit keeps its 32 lane masks from being
  // hoisted out of the loop and held in registers for the whole pass.
  auto mask_tail = [&](f32x16* s, int nvalid) __attribute__((always_inline)) {
    int lim = nvalid - 4 * lh;
    opaque(lim);
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        if (32 * b + 8 * (r >> 2) + (r & 3) >= lim) s[b][r] = -INFINITY;
  };
  // ---- online softmax of x = s * c (base-2 units; tmax already scaled) into
  // the fp16 P operand, raising m when needed.
  // score scale of this lane's P chunk cc: per 16-key group with 16-key
  // blocks, else the step's (with blocks of <= 8 keys the common factor, which
  // FULL steps use as is)
  auto chunk_scale = [&](const StepScale<G>& cs, int cc) __attribute__((always_inline)) {
    if constexpr (G == 4) return cs.c[cc];
    else return cs.c[0];
  };
  // raise the running reference m to a step's maximum tmax (base 2, already
  // reduced over the lane pair) when it exceeds m by more than kLazy
  auto raise_max = [&](float tmax, auto lazy) __attribute__((always_inline)) {
    const bool need = tmax > m_run + kLazy;
    if (__ballot(need)) {
      const float mn = need ? tmax : m_run;
      const float al = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
      l_run *= al;
      if constexpr (decltype(lazy)::value) {
        accF *= al;   // the quantised phases carry the factor instead
      } else {
#pragma unroll
        for (int db = 0; db < D / 32; db++)
#pragma unroll
          for (int r = 0; r < 16; r++) acc[db][r] *= al;
      }
      m_run = mn;
    }
  };
  // BF: the P operand in bf16 (FULL tiles), else fp16 (skip chunks)
  auto softmax = [&](f32x16* s, const StepScale<G>& cs, float tmax, auto bf) __attribute__((always_inline)) {
    constexpr bool BF = decltype(bf)::value;
    raise_max(max_lane_halves(tmax), std::false_type{});
    const float nm = -m_run;
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int tt = 0; tt < 8; tt++) {
        const int e = 8 * cc + tt;
        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 4][e & 15], chunk_scale(cs, cc), nm));
        if constexpr (BF) pb[cc][tt] = __builtin_bit_cast(_Float16, static_cast<__bf16>(x));
        else pb[cc][tt] = static_cast<_Float16>(x);
      }
    l_run += BF ? bf16_sum(pb) : half_sum(pb);
  };
  auto row_max = [&](const f32x16* s) __attribute__((always_inline)) {
    float m = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) m = __builtin_fmaxf(m, s[b][r]);
    return m;
  };
  // ---- O^T += V^T P^T of a skip chunk from region R1: the pooled V^T [D][64]
  // fp16, keys in the P.V operand's order (vt_pos)
  auto pv = [&](const unsigned char* st) __attribute__((always_inline)) {
    f16x8 va[D / 8];
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int db = 0; db < D / 32; db++)
        va[cc * (D / 32) + db] = *reinterpret_cast<const f16x8*>(r1(st) + offv[cc] + db * 32 * 128);
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int db = 0; db < D / 32; db++)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[cc * (D / 32) + db], pb[cc], acc[db], 0, 0, 0);
    pipeline_reads_mfma<D / 8, D / 16>();
  };

  // ---- O^T += V^T P^T from V rows in R1, read transposed, two 4-row reads per
  // operand (score rows 16cc + 4lh + 0..3, then + 8): a FULL step's caller V
  // against bf16 P on the bf16 MFMA (BF), or the low tier's fp16 V rows of a
  // gathered step against fp16 P on the fp16 MFMA.
  //
  // Transposing reads (ds_read_b64_tr_b16): in each 16-lane group the lanes
  // name sixteen 8-byte pieces, lane 4u + a the piece at row u, columns
  // 4a..4a+3 of a 4-row x 16-column block, and lane 4a + c then receives
  // column 4a + c of the four rows (an in-bounds probe on gfx950 confirmed this
  // lane mapping).  The A operand of P chunk cc is V^T at d = 32db + ln over
  // the score rows 16cc + 4lh + 0..3 and 16cc + 8 + 4lh + 0..3 (the keys of the
  // lane's P values, in their order), so group g = lane >> 4 reads columns
  // 32db + 16(g & 1) .. +15 of rows 16cc + 4lh (+ 8) + u.  The lane offsets
  // are formed here from an opaque lane index, so they are not held in
  // registers across the step loop.
  auto pv_rows = [&](const unsigned char* st, auto bf) __attribute__((always_inline)) {
    constexpr bool BF = decltype(bf)::value;
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const unsigned char* r = r1(st);
    int lr = lane_here();
    int offtr[D / 32];
    {
      const int u = (lr >> 2) & 3, aa = lr & 3, gg = (lr >> 4) & 1, row = 4 * (lr >> 5) + u;
#pragma unroll
      for (int db = 0; db < D / 32; db++)
        offtr[db] = row * (2 * D) + (((4 * db + 2 * gg + (aa >> 1)) ^ swzv<D>(row)) << 4) + 8 * (aa & 1);
    }
    bf16x8 va[D / 8];
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int db = 0; db < D / 32; db++) {
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(r + offtr[db] + 16 * cc * (2 * D)));
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(r + offtr[db] + (16 * cc + 8) * (2 * D)));
        va[cc * (D / 32) + db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int db = 0; db < D / 32; db++)
        if constexpr (BF)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cc * (D / 32) + db], __builtin_bit_cast(bf16x8, pb[cc]),
                                                            acc[db], 0, 0, 0);
        else
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, va[cc * (D / 32) + db]), pb[cc],
                                                           acc[db], 0, 0, 0);
    pipeline_reads2_mfma<D / 8, D / 16>();
  };

  // ---- quantised probabilities (LOW and SKIM tiles).  Scores x = s * c in
  // base 2; per row the tile maximum tm; codes E(448 * 2^(x - tm)), so the
  // maximum lands on 448; the tile's weight relative to the running reference
  // is 2^(tm - m) / 448 per code unit.  The codes stay in p8 in register
  // order (byte p = 16b + r of lane half h: score register (b, r)), which is
  // the B operand of the fp8 P.V.
  auto dump_codes = [&](int ds) __attribute__((always_inline)) {
    if constexpr (DUMP) {
      if (dsl >= 0 && ds < a.dsteps) {
        int lr = lane_here();   // opaque: the lane's term is not kept live across the kernel
        unsigned char* o = a.dump + ((static_cast<int64_t>(dsl) * a.dsteps + ds) * (32 * NW) + 32 * wave + (lr & 31)) * 64 + 32 * (lr >> 5);
        reinterpret_cast<uint4*>(o)[0] = make_uint4(p8[0], p8[1], p8[2], p8[3]);
        reinterpret_cast<uint4*>(o)[1] = make_uint4(p8[4], p8[5], p8[6], p8[7]);
      }
    } else {
      (void)ds;
    }
  };
  // codes of four scores, x = 2^(s * c - tm + log2(448)), into one dword.
  // x is at most 448 up to rounding (far below 464, where the converter
  // would stop rounding to 448), so it needs no clamp.
  // `old` is the dword's previous value: both halves are overwritten, and
  // passing the register it already occupies needs no copy.
  auto codes4 = [&](float s0, float s1, float s2, float s3, float c, float nm, int old) __attribute__((always_inline)) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(__builtin_fmaf(s0, c, nm)),
                                                  __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, nm)), old, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(__builtin_fmaf(s2, c, nm)),
                                           __builtin_amdgcn_exp2f(__builtin_fmaf(s3, c, nm)), w, true);
  };
  // 64-key tile: one maximum per row (over both lane halves); the row sum of
  // the codes from the fp8 MFMA against ones (every result register holds the
  // column sum, so each lane half adds half of it); the P.V weight split into
  // the accumulator factor and the E8M0 column scale (wr, wk)
  auto quant_soft64 = [&](f32x16* s, float c, float sv, int ds) __attribute__((always_inline)) {
    float tm = row_max(s);
    tm = max_lane_halves(tm) * c;
    raise_max(tm, std::true_type{});
    const float nm = kLog2_448 - tm;
#pragma unroll
    for (int w = 0; w < 8; w++) {
      const int b = w >> 2, r0 = 4 * (w & 3);
      p8[w] = codes4(s[b][r0], s[b][r0 + 1], s[b][r0 + 2], s[b][r0 + 3], c, nm, p8[w]);
    }
    dump_codes(ds);
    // the ones as an FP4 (E2M1 1.0 = 0x2) operand: four registers instead of eight
    const i32x8 ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
    const f32x16 rs = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, p8, f32x16{}, 4, 0, 0, 0, 0, 0);
    const float g = __builtin_amdgcn_exp2f(tm - m_run);
    l_run = __builtin_fmaf(rs[0], g * (0.5f / 448.0f), l_run);
    const float w = g * (sv * (1.0f / 448.0f));
    // w = wm 2^e, wm in [1, 2).  A weight below 2^-127 (a tile negligible
    // against the running reference) leaves accF and adds its codes at the
    // smallest scale, 2^-127.
    const int e = __builtin_amdgcn_frexp_expf(w) - 1;
    const float wm = __builtin_amdgcn_frexp_mantf(w) * 2.0f;
    const bool tiny = e < -127 || !(w > 0.0f);
    wr = tiny ? 1.0f : accF * __builtin_amdgcn_rcpf(wm);
    accF = tiny ? accF : wm;
    wk = tiny ? 0 : e + 127;
  };
  // 16-key blocks: one maximum per block (chunk cc of the lane over both lane
  // halves), and the fp16 P.V operand decode(code) * 2^(tm_block - m) / 448
  auto quant_soft_g = [&](f32x16* s, const StepScale<G>& cs, int ds) __attribute__((always_inline)) {
    float tb[4];
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < 8; r++) m = __builtin_fmaxf(m, s[cc >> 1][8 * (cc & 1) + r]);
      tb[cc] = max_lane_halves(m * chunk_scale(cs, cc));
    }
    float tmax = __builtin_fmaxf(__builtin_fmaxf(tb[0], tb[1]), __builtin_fmaxf(tb[2], tb[3]));
    raise_max(max_lane_halves(tmax), std::false_type{});
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {
      const bool live = tb[cc] > -INFINITY;   // a slot past the list's end has no keys
      const float nm = live ? kLog2_448 - tb[cc] : 0.0f;
      const float gw = live ? __builtin_amdgcn_exp2f(tb[cc] - m_run) * (1.0f / 448.0f) : 0.0f;
      const float c = chunk_scale(cs, cc);
      const int b = cc >> 1, r0 = 8 * (cc & 1);
#pragma unroll
      for (int j = 0; j < 2; j++) {
        // (0, not the register's old codes, as the kept half: p8 is then not
        // live between steps)
        const int w = codes4(s[b][r0 + 4 * j], s[b][r0 + 4 * j + 1], s[b][r0 + 4 * j + 2], s[b][r0 + 4 * j + 3], c, nm, 0);
        p8[2 * cc + j] = w;
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        pb[cc][4 * j] = static_cast<_Float16>(lo.x * gw);
        pb[cc][4 * j + 1] = static_cast<_Float16>(lo.y * gw);
        pb[cc][4 * j + 2] = static_cast<_Float16>(hi.x * gw);
        pb[cc][4 * j + 3] = static_cast<_Float16>(hi.y * gw);
      }
    }
    dump_codes(ds);
    l_run += half_sum(pb);
  };
  // Blocks of BK <= 8 keys: the lane's slot u holds its P values (flat
  // register index 16b + r) u BK .. u BK + BK - 1, and is slot
  // slotg(row of its first P value) of the step.  Scores are scaled in place
  // by their slot's scale, then per slot the maximum tb, codes
  // E(448 * 2^(x - tb)) and the fp16 P.V operand decode(code) * 2^(tb - m) / 448.
  // One-key blocks: the code is 448 for every live key, so P is 2^(x - m).
  auto quant_soft_s = [&](f32x16* s, const StepScale<G>& cs, int ds) __attribute__((always_inline)) {
    constexpr int NS = BK <= 8 ? 32 / BK : 1;   // (instances with larger blocks never call it)
    float tb[NS];
#pragma unroll
    for (int u = 0; u < NS; u++) {
      const int f0 = u * BK, b = f0 >> 4, r0 = f0 & 15;
      const int slot = slotg<BK>(32 * b + 8 * (r0 >> 2) + (r0 & 3)) + (8 / BK) * lh;
      const float c = cs.c[0] * __shfl(cs.kv, slot, 64);
      float m = -INFINITY;
#pragma unroll
      for (int z = 0; z < BK; z++) {
        s[b][r0 + z] *= c;
        m = __builtin_fmaxf(m, s[b][r0 + z]);
      }
      tb[u] = m;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < NS; u++) tmax = __builtin_fmaxf(tmax, tb[u]);
    raise_max(max_lane_halves(tmax), std::false_type{});
    if constexpr (BK == 1) {
#pragma unroll
      for (int w = 0; w < 8; w++) {
        int code = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int f = 4 * w + j;
          const float x = s[f >> 4][f & 15];
          const bool live = x > -INFINITY;
          pb[f >> 3][f & 7] = static_cast<_Float16>(live ? __builtin_amdgcn_exp2f(x - m_run) : 0.0f);
          code |= (live ? 0x7E : 0) << (8 * j);   // E4M3 448
        }
        p8[w] = code;
      }
    } else {
      float nm[NS], gw[NS];
#pragma unroll
      for (int u = 0; u < NS; u++) {
        const bool live = tb[u] > -INFINITY;   // a slot past the list's end has no keys
        nm[u] = live ? kLog2_448 - tb[u] : 0.0f;
        gw[u] = live ? __builtin_amdgcn_exp2f(tb[u] - m_run) * (1.0f / 448.0f) : 0.0f;
      }
#pragma unroll
      for (int w = 0; w < 8; w++) {
        const int f = 4 * w, b = f >> 4, r = f & 15;
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; j++) x[j] = __builtin_amdgcn_exp2f(s[b][r + j] + nm[(f + j) / BK]);
        const int lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);   // p8 not live between steps
        const int code = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo2, true);
        p8[w] = code;
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(code, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(code, true);
        const float dv[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int j = 0; j < 4; j++) pb[(f + j) >> 3][(f + j) & 7] = static_cast<_Float16>(dv[j] * gw[(f + j) / BK]);
      }
    }
    dump_codes(ds);
    l_run += half_sum(pb);
  };
  // ---- acc = acc * wr + V8^T (P8^T 2^(wk - 127)) on the fp8 MFMA (64-key LOW
  // and SKIM tiles): row d = 32db + ln of the staged E4M3 V^T, bytes 32lh ..
  // 32lh + 31; the column (query) scale is the B operand's E8M0 scale
  auto pv8 = [&](const unsigned char* st) __attribute__((always_inline)) {
    i32x8 va[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; db++) {
      const uint4 lo = *reinterpret_cast<const uint4*>(r1(st) + offv8[0] + db * 32 * 64);
      const uint4 hi = *reinterpret_cast<const uint4*>(r1(st) + offv8[1] + db * 32 * 64);
      va[db] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int db = 0; db < D / 32; db++) {
#pragma unroll
      for (int r = 0; r < 16; r++) acc[db][r] *= wr;
      acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[db], p8, acc[db], 0, 0, 0, 127, 0, wk);
    }
  };
  // a kept tile (FULL: bf16 scores, LOW: E4M3 scores): masks and softmax of
  // its scores s
  auto kept_soft = [&](auto low_tag, int t, f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) {
    constexpr bool LOW = decltype(low_tag)::value;
    if constexpr (G == 1) {
      const int J = list_at(t);
      if (J == dm.Nk - 1) mask_tail(s, dm.N - 64 * J);
      if constexpr (LOW) quant_soft64(s, c.c[0], c.v, t - tLow);
      else softmax(s, c, row_max(s) * c.c[0], std::true_type{});
    } else {
      // Lists are ascending, so a partial group or the ragged last block only
      // occurs in the last step of the phase.
      if (t == (!LOW ? tLow - 1 : (SKIM && t >= tSk) ? nSteps - 1 : tSk - 1)) {
        const int i0 = list_idx(t, 0), e = list_end(t);
        if constexpr (G == 4) {
          // Register (b, r) is key 8((r >> 2) & 1) + 4lh + r % 4 of 16-key
          // block 2b + r / 8.  Valid keys of each block: 0 past the list end,
          // fewer in block Nk - 1.
          int ql[4];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int Jg = (int)slist[i0 + q < e ? i0 + q : i0];
            ql[q] = (i0 + q >= e ? 0 : Jg == dm.Nk - 1 ? dm.N - BK * Jg : BK) - 4 * lh;
            opaque(ql[q]);
          }
#pragma unroll
          for (int b = 0; b < 2; b++)
#pragma unroll
            for (int r = 0; r < 16; r++)
              if (8 * ((r >> 2) & 1) + (r & 3) >= ql[2 * b + (r >> 3)]) s[b][r] = -INFINITY;
        } else {
          // the lane's slot u: P values u BK + z hold keys z = 0 .. BK-1 (the
          // lane half from the hardware lane index: not held across the loop)
          const int lhs = lane_here() >> 5;
#pragma unroll
          for (int u = 0; u < 32 / BK; u++) {
            const int f0 = u * BK, b = f0 >> 4, r0 = f0 & 15;
            const int slot = slotg<BK>(32 * b + 8 * (r0 >> 2) + (r0 & 3)) + (8 / BK) * lhs;
            const bool in = i0 + slot < e;
            const int Js = in ? (int)slist[i0 + slot] : 0;
            int lim = !in ? 0 : Js == dm.Nk - 1 ? dm.N - BK * Js : BK;
            opaque(lim);
#pragma unroll
            for (int z = 0; z < BK; z++)
              if (z >= lim) s[b][r0 + z] = -INFINITY;
          }
        }
      }
      if constexpr (LOW && G == 4) {
        quant_soft_g(s, c, t - tLow);
      } else if constexpr (LOW) {
        quant_soft_s(s, c, t - tLow);
      } else {
        float tmax = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < 4; cc++) {
          float m = -INFINITY;
#pragma unroll
          for (int r = 0; r < 8; r++) m = __builtin_fmaxf(m, s[cc >> 1][8 * (cc & 1) + r]);
          tmax = __builtin_fmaxf(tmax, m * chunk_scale(c, cc));
        }
        softmax(s, c, tmax, std::true_type{});
      }
    }
  };
  // a kept tile staged in `st`: scores, softmax, P.V
  // low_scores(st, s): a LOW step's scores (E4M3 or refined); unused for FULL
  auto kept_step = [&](auto low_tag, int t, const unsigned char* st, const StepScale<G>& c, auto low_scores) __attribute__((always_inline)) {
    constexpr bool LOW = decltype(low_tag)::value;
    f32x16 s[2] = {f32x16{}, f32x16{}};
    if constexpr (LOW) low_scores(st, s);
    else scores_bf16(st, s);
    kept_soft(low_tag, t, s, c);
    if constexpr (LOW && G == 1) pv8(st);
    else pv_rows(st, std::integral_constant<bool, !LOW>{});
  };
  // a SKIM step: mask and quantised probabilities of its scores s (with
  // gathered blocks as a LOW step's, the scale factor being the step's)
  auto skim_soft = [&](int t, f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) {
    if constexpr (G == 1) {
      const int J = list_at(t);
      if (J == dm.Nk - 1) mask_tail(s, dm.N - 64 * J);
      quant_soft64(s, c.c[0], c.v, t - tLow);
    } else {
      kept_soft(std::true_type{}, t, s, c);
    }
  };
  auto skim_step = [&](int t, const unsigned char* st, const StepScale<G>& c, const i32x8* q4, const int* q4s) __attribute__((always_inline)) {
    f32x16 s[2] = {f32x16{}, f32x16{}};
    scores_fp4(st, s, q4, q4s);
    skim_soft(t, s, c);
    if constexpr (G == 1) pv8(st);
    else pv_rows(st, std::false_type{});
  };
  // pooled keys of a chunk of 64 skipped-candidate blocks: scores only (hi
  // part from R0, lo part from R1), then the bias and the softmax
  auto skip_S = [&](const unsigned char* st, f32x16* s) __attribute__((always_inline)) {
    scores_bf16(st, s);
    // low half of kbar; with one-key blocks the mean is the key itself, a bf16
    // value, so the low half is zero and its pass is left out
    if constexpr (BK > 1) scores_bf16(r1(st), s);
  };
  auto skip_soft = [&](int t, f32x16* s) __attribute__((always_inline)) {
    // bias log2(n_J) for the row's skipped blocks, -inf for the others.  Key
    // 32b + 8(r/4) + 4lh + r%4 of the chunk is bit 32b + 8(r/4) + r%4 of the
    // chunk's mask shifted right by 4lh.
    const int ci = t >> 1;
    const uint64_t msk = smask[ci] >> (4 * lh);
    const uint32_t mw[2] = {static_cast<uint32_t>(msk), static_cast<uint32_t>(msk >> 32)};
    // position of the ragged last block inside this lane's view of the chunk
    // (only the chunk holding block Nk - 1 can match)
    const int lastpos = dm.Nk - 1 - 64 * schunk[ci] - 4 * lh;
    const float lglast = __log2f(static_cast<float>(dm.N - (dm.Nk - 1) * BK));
    constexpr float lgfull = BK == 64 ? 6.0f : BK == 16 ? 4.0f : BK == 8 ? 3.0f : BK == 4 ? 2.0f : BK == 2 ? 1.0f : 0.0f;   // log2(BK)
    float tmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int pos = 8 * (r >> 2) + (r & 3);
        const bool sk = (mw[b] >> pos) & 1u;
        const float lg = 32 * b + pos == lastpos ? lglast : lgfull;
        s[b][r] = sk ? __builtin_fmaf(s[b][r], cF, lg) : -INFINITY;
        tmax = __builtin_fmaxf(tmax, s[b][r]);
      }
    StepScale<G> one;
#pragma unroll
    for (int g = 0; g < StepScale<G>::N; g++) one.c[g] = 1.0f;
    softmax(s, one, tmax, std::false_type{});
  };
  auto skip_scores = [&](int t, const unsigned char* st) __attribute__((always_inline)) {
    f32x16 s[2] = {f32x16{}, f32x16{}};
    skip_S(st, s);
    skip_soft(t, s);
  };

  // ---- the step loop, in phases (skip chunks as score / P.V pairs, FULL,
  // LOW, SKIM).  Step t computes from stage t & 1 while step t+1's DMA fills the
  // other stage; the explicit vmcnt(0) + barrier publishes it.  The parity is
  // a compile-time tag, so each stage is a distinct array at every access.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  StepScale<G> cA{}, cB{};   // per-stage score scale
  auto stg = [&](auto p) __attribute__((always_inline)) -> unsigned char* {
    if constexpr (decltype(p)::value) return stB;
    else return stA;
  };
  auto scl = [&](auto p) __attribute__((always_inline)) -> StepScale<G>& {
    if constexpr (decltype(p)::value) return cB;
    else return cA;
  };
  auto flip = [](auto p) { return std::integral_constant<int, 1 - decltype(p)::value>{}; };
  auto next = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);   // the step's work stays ahead of its closing wait
    wait_vm0_lgkm0();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    refresh();
  };
  constexpr int kSk = SKIM ? 1 << kSkim : 0;
  using KAll = std::integral_constant<int, 15 | kSk>;
  using KAfterFull = std::integral_constant<int, (1 << kFull) | (1 << kLow) | kSk>;
  using KSkipS = std::integral_constant<int, 1 << kSkipS>;
  using KSkipPV = std::integral_constant<int, 1 << kSkipPV>;
  using KAfterSkip = std::integral_constant<int, (1 << kSkipS) | (1 << kFull) | (1 << kLow) | kSk>;
  using KLow = std::integral_constant<int, (1 << kLow) | kSk>;
  using KSkimOnly = std::integral_constant<int, kSk>;
  // the E4M3 copy of this lane's Q (32 bytes per fp8 instruction i = bf16
  // chunks 4i..4i+3), from the bf16 registers
  auto make_q8 = [&](i32x8* q8reg) __attribute__((always_inline)) {
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
  };
  // the MXFP4 copy of this lane's Q row (channels 64i + 32lh .. +31 for
  // instruction i, one E8M0 scale each), from Q in memory
  auto make_q4 = [&](i32x8* q4reg, int* q4s, i32x8* q4rreg = nullptr, int* q4rs = nullptr) __attribute__((always_inline)) {
    // buffer loads through a resource over the head's rows: a row past N
    // reads as zeros without a branch
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(a.q + toff, (uint32_t)dm.N * (uint32_t)dm.sn * 2);
    // the row from an opaque lane index: the Q loads' row term is not held
    // live from the kernel's start to here
    int lr = lane_here();
    const int qoff = ((I * (32 * NW) + wave * 32 + (lr & 31)) * (int)dm.sn + 32 * (lr >> 5)) * 2;
    auto load32 = [&](int i, float* x) __attribute__((always_inline)) {   // channels 64i + 32lh .. +31
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint4 raw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rQ, qoff + (64 * i + 8 * j) * 2, 0, 0));
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; e++) x[8 * j + e] = __uint_as_float(e & 1 ? (wd[e >> 1] & 0xffff0000u) : (wd[e >> 1] << 16));
      }
    };
    auto encode32 = [&](const float* x, int& ex) __attribute__((always_inline)) {   // MXFP4 codes of 32 values
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; e++) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[e]));
      ex = mx4_exponent(amax);
      uint32_t pk[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 32; e++) pk[e >> 3] |= e2m1_code(ldexpf(x[e], -ex)) << (4 * (e & 7));
      return i32x8{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], 0, 0, 0, 0};
    };
#pragma unroll
    for (int i = 0; i < D / 64; i++) {
      float x[32];
      load32(i, x);
      int ex;
      q4reg[i] = encode32(x, ex);
      q4s[i] = ex + 127;
    }
    if constexpr (REFINE) {
      // the residual x - code 2^e (exact in float32), one 32-channel chunk at
      // a time from a second read of Q: computed in the first pass it kept
      // twice the values live and the register allocator spilled
#pragma unroll
      for (int i = 0; i < D / 64; i++) {
        __builtin_amdgcn_sched_barrier(0);
        float x[32];
        load32(i, x);
        const int ex = q4s[i] - 127;
#pragma unroll
        for (int e = 0; e < 32; e++)
          x[e] -= ldexpf(e2m1_value((static_cast<uint32_t>(q4reg[i][e >> 3]) >> (4 * (e & 7))) & 15u), ex);
        int er;
        q4rreg[i] = encode32(x, er);
        q4rs[i] = er + 127;
      }
    } else {
      (void)q4rreg;
      (void)q4rs;
    }
  };


  if constexpr (!SPLIT) {
    if (nSteps > 0) issue(KAll{}, 0, stA, cA);
    wait_vm0();
    __syncthreads();
    int t = 0;
    // a phase of single steps [t, end): two copies of the body, one per parity
    auto run_phase = [&](int end, auto body) __attribute__((always_inline)) {
      while (t < end) {
        if ((t & 1) == 0) {
          body(P0{}, t);
          if (++t == end) break;
        }
        body(P1{}, t);
        ++t;
      }
    };
    // skip pairs first, from step 0 (even parity)
    for (; t < nS2; t += 2) {
      issue(KSkipPV{}, t + 1, stB, cB);
      skip_scores(t, stA);
      next();
      if (t + 2 < nSteps) issue(KAfterSkip{}, t + 2, stA, cA);
      pv(stB);
      next();
    }
    run_phase(tLow, [&](auto p, int tt) __attribute__((always_inline)) {
      if (tt + 1 < nSteps) issue(KAfterFull{}, tt + 1, stg(flip(p)), scl(flip(p)));
      kept_step(std::false_type{}, tt, stg(p), scl(p), nullptr);
      next();
    });
    if (t < tSk) {   // LOW tiles remain: make the E4M3 copy of Q (32 bytes per
                     // fp8 instruction i = bf16 chunks 4i..4i+3), or for the
                     // refined tier the MXFP4 copy of Q and of its residual
      i32x8 q8reg[D / 64];
      i32x8 q4reg[REFINE ? D / 64 : 1], q4rreg[REFINE ? D / 64 : 1];
      int q4s[REFINE ? D / 64 : 1], q4rs[REFINE ? D / 64 : 1];
      if constexpr (REFINE) make_q4(q4reg, q4s, q4rreg, q4rs);
      else make_q8(q8reg);
      // a LOW step's scores from the K operands staged in `st`
      auto low_scores = [&](const unsigned char* st, f32x16* sc) __attribute__((always_inline)) {
        if constexpr (REFINE) scores_refine(st, sc, q4reg, q4s, q4rreg, q4rs);
        else scores_fp8(st, sc, q8reg);
      };
      if constexpr (G == 1) {
        // Software pipeline: step t+1's score MFMAs are issued ahead of step
        // t's softmax, so the matrix core works while the VALU quantises the
        // probabilities.  Entering iteration t: the scores of step t are in
        // registers (sE for even t, sO for odd t), step t's V is in R1 of its
        // stage, step t+1's R0 half (its K codes) has landed in the other
        // stage.  Iteration t refills R0 of step t's stage with step t+2's K
        // half and R1 of the other stage with step t+1's V half, then scores
        // step t+1 and finishes step t.
        //
        // List window: lane l holds the key block, score scale and value
        // scale of step tLow + wb + l (the LOW entries, then the SKIM ones),
        // read once per 32 steps; a step takes its entries with readlane, so
        // it waits on neither an LDS read of the list nor a scalar-memory
        // load of the scales.
        int wb = 0, jw, jn = 0;
        float cw, vw, cn = 0.0f, vn = 0.0f;
        auto window = [&](int base, int& jx, float& cx, float& vx) __attribute__((always_inline)) {
          const int i = nF + base + lane;
          const int J = i < nK + nSk ? (int)slist[i] : 0;
          jx = J;
          cx = REFINE ? cF : sq * skp[J] * cF;   // refined: the fp4 scales are inside the MFMA
          vx = svp[J];
        };
        auto rl = [](int x, int l) __attribute__((always_inline)) { return __builtin_amdgcn_readlane(x, l); };
        auto rlf = [](float x, int l) __attribute__((always_inline)) {
          return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
        };
        auto low_k = [&](int J, unsigned char* st) __attribute__((always_inline)) {   // the K operands of block J into R0
          if constexpr (REFINE) {
            refine_k(J, st);
          } else {
#pragma unroll
            for (int i = 0; i < NI8; i++) {
              const int k = wave + NW * i;
              dma16(rS, st + k * 1024, voffK8, (int)SL.k8 + J * 64 * D + k * 1024);
            }
          }
        };
        using PartK = std::integral_constant<int, 1>;
        window(0, jw, cw, vw);
        f32x16 sE[2], sO[2];
        auto sreg = [&](auto p) __attribute__((always_inline)) -> f32x16* {
          if constexpr (decltype(p)::value) return sO;
          else return sE;
        };
        // prologue: step t is staged whole; stage the K half of step t+1
        auto prologue = [&](auto p) __attribute__((always_inline)) {
          if (t + 1 < tSk) low_k(rl(jw, 1), stg(flip(p)));
          else if (t + 1 < nSteps) issue_part(KLow{}, PartK{}, t + 1, stg(flip(p)), scl(flip(p)));   // a SKIM step
          f32x16* sc = sreg(p);
          sc[0] = f32x16{};
          sc[1] = f32x16{};
          low_scores(stg(p), sc);
          next();
        };
        if (t & 1) prologue(P1{});
        else prologue(P0{});
        run_phase(tSk, [&](auto p, int tt) __attribute__((always_inline)) {
          // The window slides by 32 steps: at o = 61 the next one is loaded
          // (landed by the step's closing wait), at o = 62 it is taken.  Both
          // branches stay ahead of the step's compute, which is then one basic
          // block up to its closing barrier.
          const int k = tt - tLow;
          if (k - wb == 62) {
            jw = jn;
            cw = cn;
            vw = vn;
            wb += 32;
          }
          const int o = k - wb;   // o <= 61: steps k .. k+2 are in the window
          if (o == 61) window(wb + 32, jn, cn, vn);
          const int J = rl(jw, o);
          const float c = rlf(cw, o), sv = rlf(vw, o);
          if (tt + 2 < tSk) low_k(rl(jw, o + 2), stg(p));
          else if (tt + 2 < nSteps) issue_part(KLow{}, PartK{}, tt + 2, stg(p), scl(p));   // a SKIM step
          if (tt + 1 < nSteps) load_v8(r1(stg(flip(p))), rl(jw, o + 1));   // LOW and SKIM: E4M3 V^T
          f32x16* sc = sreg(p);
          if (J == dm.Nk - 1) mask_tail(sc, dm.N - 64 * J);   // the ragged last block (a branch)
          // (the last iteration scores a stale, in-bounds R0 and drops the
          // result: unconditional, the score MFMAs share a block with the
          // softmax and the scheduler can interleave them)
          f32x16* sn = sreg(flip(p));
          sn[0] = f32x16{};
          sn[1] = f32x16{};
          low_scores(stg(flip(p)), sn);
          quant_soft64(sc, c, sv, k);
          pv8(stg(p));
          if constexpr (REFINE) schedule_refine_step<D>();
          else schedule_low_step<D>();
          next();
        });
      } else {
        run_phase(tSk, [&](auto p, int tt) __attribute__((always_inline)) {
          if (tt + 1 < nSteps) issue(KLow{}, tt + 1, stg(flip(p)), scl(flip(p)));
          kept_step(std::true_type{}, tt, stg(p), scl(p), low_scores);
          next();
        });
      }
    }
    if constexpr (SKIM) {
      if (t < nSteps) {   // SKIM tiles remain: the MXFP4 copy of this lane's Q row,
                          // channels 64i + 32lh .. +31 for instruction i
        i32x8 q4reg[D / 64];
        int q4s[D / 64];
        make_q4(q4reg, q4s);
        run_phase(nSteps, [&](auto p, int tt) __attribute__((always_inline)) {
          if (tt + 1 < nSteps) issue(KSkimOnly{}, tt + 1, stg(flip(p)), scl(flip(p)));
          skim_step(tt, stg(p), scl(p), q4reg, q4s);
          next();
        });
      }
    }

  } else {
    // ---- single stage (two-wave workgroups).  Step t's R0 half is staged
    // when it starts and its R1 half may still be in flight.  After the
    // score reads the R0 half of step t+1 is issued, after the P.V reads the
    // R1 half, so before P.V this wave's outstanding DMA is [R1 of t, R0 of
    // t+1] and the wait leaves R0 of t+1's instructions in flight.
    using PA = std::integral_constant<int, 1>;
    using PB = std::integral_constant<int, 2>;
    auto bar = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // this wave's R0-half instructions for step u (none past the last step)
    auto a_count = [&](int u) -> int {
      if (u >= nSteps) return 0;
      const int k = step_kind(u);
      if (k == kFull || k == kSkipS) return NI16;
      // LOW: refined, K rows and residual rows, one scale-word load each from
      // the first and last wave; with blocks of <= 8 keys the E4M3 K rows and
      // the per-lane load of the slots' scales
      if (k == kLow)
        return REFINE ? 2 * ((D / 32 - wave + NW - 1) / NW) + (wave == 0 ? 1 : 0) + (wave == NW - 1 ? 1 : 0)
                      : NI8 + (G >= 8 ? 1 : 0);
      if (k == kSkipPV) return 0;
      return (D / 32 - wave + NW - 1) / NW + (wave == 0 ? 1 : 0);   // SKIM: K rows and the scale words
    };
    if (nSteps > 0) {
      issue_part(KAll{}, PA{}, 0, stA, cA);
      issue_part(KAll{}, PB{}, 0, stA, cA);
    }
    wait_vm0();
    __syncthreads();
    int t = 0;
    // One step.  S_fn(s): its scores from the stage; soft_fn(s, c): masks and
    // softmax.  HS: the step scores; HP: it runs P.V; U1: its scores also
    // read R1 (a skip chunk's lo half); Q8PV: which P.V it runs.
    auto split_step = [&](auto nk, auto hs, auto hp, auto u1, auto q8pv, auto S_fn, auto soft_fn) __attribute__((always_inline)) {
      constexpr bool HS = decltype(hs)::value, HP = decltype(hp)::value, U1 = decltype(u1)::value;
      // P.V: 1 on the fp8 MFMA (quantised 64-key steps), 2 the FULL one on the
      // caller's V rows, 3 the fp16 one on the low tier's V rows (gathered
      // steps), 0 the fp16 one on the pooled V^T (skip chunks)
      constexpr int PVK = static_cast<int>(decltype(q8pv)::value);
      const bool more = t + 1 < nSteps;
      const StepScale<G> cur = cA;   // issuing step t+1's R0 half rewrites cA
      f32x16 s[2] = {f32x16{}, f32x16{}};
      if constexpr (U1) {            // R1 of this step as well
        wait_vm0();
        bar();
      }
      if constexpr (HS) S_fn(s);
      wait_lgkm0();                  // every wave's R0 (and R1) reads have returned
      bar();
      if (more) issue_part(nk, PA{}, t + 1, stA, cA);
      if constexpr (HS) soft_fn(s, cur);
      if constexpr (HP) {
        wait_vm_n(a_count(t + 1));   // R1 of step t landed in every wave
        bar();
        if constexpr (PVK == 1) pv8(stA);
        else if constexpr (PVK == 2) pv_rows(stA, std::true_type{});
        else if constexpr (PVK == 3) pv_rows(stA, std::false_type{});
        else pv(stA);
      }
      wait_vm0_lgkm0();              // R0 of step t+1 landed, this wave's R1 reads returned
      bar();
      refresh();
      if (more) issue_part(nk, PB{}, t + 1, stA, cA);
      ++t;
    };
    using T0 = std::false_type;
    using T1 = std::true_type;
    auto no_S = [&](f32x16*) {};
    auto no_soft = [&](f32x16*, const StepScale<G>&) {};
    while (t < nS2) {
      if ((t & 1) == 0)
        split_step(KSkipPV{}, T1{}, T0{}, std::integral_constant<bool, (BK > 1)>{}, T0{},
                   [&](f32x16* s) __attribute__((always_inline)) { skip_S(stA, s); },
                   [&](f32x16* s, const StepScale<G>&) __attribute__((always_inline)) { skip_soft(t, s); });
      else
        split_step(KAfterSkip{}, T0{}, T1{}, T0{}, T0{}, no_S, no_soft);
    }
    while (t < tLow)
      split_step(KAfterFull{}, T1{}, T1{}, T0{}, std::integral_constant<int, 2>{},
                 [&](f32x16* s) __attribute__((always_inline)) { scores_bf16(stA, s); },
                 [&](f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) { kept_soft(T0{}, t, s, c); });
    if (t < tSk) {
      i32x8 q8reg[D / 64];
      i32x8 q4reg[REFINE ? D / 64 : 1], q4rreg[REFINE ? D / 64 : 1];
      int q4s[REFINE ? D / 64 : 1], q4rs[REFINE ? D / 64 : 1];
      if constexpr (REFINE) make_q4(q4reg, q4s, q4rreg, q4rs);
      else make_q8(q8reg);
      while (t < tSk)
        split_step(KLow{}, T1{}, T1{}, T0{}, std::integral_constant<int, G == 1 ? 1 : 3>{},
                   [&](f32x16* s) __attribute__((always_inline)) {
                     if constexpr (REFINE) scores_refine(stA, s, q4reg, q4s, q4rreg, q4rs);
                     else scores_fp8(stA, s, q8reg);
                   },
                   [&](f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) { kept_soft(T1{}, t, s, c); });
    }
    if constexpr (SKIM) {
      if (t < nSteps) {
        i32x8 q4reg[D / 64];
        int q4s[D / 64];
        make_q4(q4reg, q4s);
        while (t < nSteps)
          split_step(KSkimOnly{}, T1{}, T1{}, T0{}, std::integral_constant<int, G == 1 ? 1 : 3>{},
                     [&](f32x16* s) __attribute__((always_inline)) { scores_fp4(stA, s, q4reg, q4s); },
                     [&](f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) { skim_soft(t, s, c); });
      }
    }
  }

  // ---- epilogue: O = acc / l.  The row's address is formed again here from
  // an opaque lane index: shared with the Q loads, it stayed live across the
  // kernel and spilled in the two-wave instances.
  // the row's normaliser: this lane's l plus the other lane half's.  The swap
  // returns (lanes 0-31: own, other) and (lanes 32-63: other, own).
  const auto lsw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float L = __uint_as_float(lsw2[0]) + __uint_as_float(lsw2[1]);
  const float scale = accF / L;
  const int lo = lane_here() & 31;
  const int orow = I * (32 * NW) + wave * 32 + lo;
  if (orow < dm.N) {
    if (a.out_fp32) {
      float* o = reinterpret_cast<float*>(a.o) + toff + (int64_t)orow * dm.sn;
#pragma unroll
      for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int d0 = 32 * db + 8 * j + 4 * lh;
          *reinterpret_cast<float4*>(o + d0) = make_float4(acc[db][4 * j] * scale, acc[db][4 * j + 1] * scale,
                                                           acc[db][4 * j + 2] * scale, acc[db][4 * j + 3] * scale);
        }
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(a.o) + toff + (int64_t)orow * dm.sn;
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

// The launches of one key-block size: every (d, waves, dump, SKIM, refine)
// instance with BK-key blocks.  Each key-block size is instantiated in its own
// translation unit (k3_bk*.hip) so that the instances compile in parallel.
template <int BK, int D, int NW, bool DUMP>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  if (a.skim && a.refine) return hipErrorInvalidValue;
  if (a.d.Nk > kMaxNk || a.list_cap < 1 || a.list_cap > a.d.Nk) return hipErrorInvalidValue;
  if (DUMP && (!a.dslot || !a.dump || a.dsteps < 1)) return hipErrorInvalidValue;
  const size_t lds = ((size_t)a.list_cap * 2 + 15) / 16 * 16;   // the row's list (dynamic LDS)
  const dim3 grid(a.d.BH * a.d.Nq), block(NW * 64);
  if (a.skim)
    hipLaunchKernelGGL((k3_attn<D, NW, BK, true, DUMP, false>), grid, block, lds, s, a);
  else if (a.refine)
    hipLaunchKernelGGL((k3_attn<D, NW, BK, false, DUMP, true>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((k3_attn<D, NW, BK, false, DUMP, false>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int BK>
hipError_t launch_bk(const AttnArgs& a, hipStream_t s) {
  if (a.d.Bk != BK) return hipErrorInvalidValue;
  const int D = a.d.D, BQ = a.d.Bq;
  const bool dump = a.dump != nullptr;
  if (D == 128 && BQ == 128) return dump ? launch_one<BK, 128, 4, true>(a, s) : launch_one<BK, 128, 4, false>(a, s);
  if (D == 128 && BQ == 64) return dump ? launch_one<BK, 128, 2, true>(a, s) : launch_one<BK, 128, 2, false>(a, s);
  if (D == 64 && BQ == 128) return dump ? launch_one<BK, 64, 4, true>(a, s) : launch_one<BK, 64, 4, false>(a, s);
  if (D == 64 && BQ == 64) return dump ? launch_one<BK, 64, 2, true>(a, s) : launch_one<BK, 64, 2, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace tattn
