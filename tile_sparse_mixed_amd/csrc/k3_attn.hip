// K3: the fused three-tier attention pass ("Triage": skip / low precision /
// full tiles executed in a single pass; "APT": dual-precision compute units
// and a tile dataflow; "FG-Attn": dense work only on kept tiles).
//
// One workgroup per (b, h, query block I) of BQ = 32 * NW rows; wave w owns
// rows 32w..32w+31 and computes S^T = K Q^T, so each lane holds one query
// column and its softmax statistics stay inside the lane pair (l, l^32).
// The workgroup walks a sequence of 64-key steps:
//   FULL      a kept tile: K (bf16, the caller's tensor) and V^T (fp16
//             copy, exact for bf16 values in fp16's normal range); S^T on
//             v_mfma_f32_32x32x16_bf16, O^T += V^T P^T on the fp16 variant
//             (P in [0, 2^8] keeps 3 more mantissa bits than bf16 would),
//   LOW       a low-precision tile: S^T on v_mfma_f32_32x32x64_f8f6f4 from the
//             E4M3 copies of Q and K scaled by sq*sk; P.V against the fp16
//             dequantised E4M3 V,
//   SKIP_S    64 pooled keys kbar_J of one chunk of 64 key blocks, as a bf16
//             hi + lo pair (two MFMAs: ~2^-17 precision), each scored with a
//             log2(n_J) bias if J is skipped in this row and -inf otherwise
//             ("Triage": a skipped tile is one score weighted by n_J),
//   SKIP_PV   the same chunk's block means vbar_J (fp16, transposed) for P.V,
//   SKIM      (instances with SKIM = true, 64-key blocks) a 4-bit tile: S^T on
//             the same instruction with MXFP4 operands and their E8M0 block
//             scales ("Triage": skimming in 4 bits); P.V against the fp16
//             dequantised MXFP4 V.
// Skipped blocks are visited as whole chunks of 64 (contiguous operands),
// masked to the row's SKIP set; chunks with no skipped block are not visited.
// With 16-key blocks ("FG-Attn": M x N tiles with a small N) a FULL or LOW
// step gathers up to four consecutive entries of the row's list into one
// 64-key step: K and E4M3 K rows per DMA instruction, V^T columns per lane (a
// 16-key block keeps its within-group key order at any column group).  With
// 8-key blocks a step gathers eight: each block's K rows go to the score rows
// whose P values form one 8-key chunk of the P.V operand (slot8 / kk8), so the
// block's V^T row is one 16-byte load in natural key order.
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
#include <type_traits>

#include "tattn_device.hpp"
#include "tattn_internal.hpp"

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
template <int D>
__device__ inline int offK8(int row, int ch) {                                  // [64][D] bytes
  return D == 128 ? row * 128 + ((ch ^ swz128(row)) << 4) : row * 64 + ((ch ^ swz64(row)) << 4);
}

// score scale of each 16-key group of a staged step (one value for 64-key
// blocks); with 8-key blocks, of this lane's four P chunks (slots 2 cc + lane
// half), held per lane so the eight slot scales need no scalar registers
template <int G>
struct StepScale {
  static constexpr int N = G == 8 ? 4 : G;
  float c[N];
};

// SKIM: the instance also runs the SKIM tier (64-key blocks only); the other
// instances carry none of its code.
template <int D, int NW, int BK, bool SKIM>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2)))
void k3_attn(AttnArgs a) {
  static_assert(BK == 64 || BK == 16 || BK == 8, "key blocks are 64, 16 or 8 keys");
  static_assert(!SKIM || BK == 64, "the SKIM tier runs on 64-key blocks");
  constexpr int G = 64 / BK;          // key blocks per 64-key step
  constexpr int STAGE = 256 * D;      // bytes: region R0 = [0, 128D), R1 = [128D, 256D)
  constexpr int R1 = 128 * D;
  // Two-wave workgroups (64-row query blocks) keep ONE stage and refill its
  // halves in turn: the K half of step t+1 while step t runs its softmax and
  // P.V, the V half while step t+1 scores.  That halves their LDS, so a CU
  // holds four of them (two waves per SIMD) instead of two (one per SIMD).
  // The halves are then two arrays (stA = R0, stB = R1), so that the
  // compiler's wait insertion sees a DMA into one half never alias reads of
  // the other.
  constexpr bool SPLIT = NW == 2;
  __shared__ __attribute__((aligned(1024))) unsigned char stA[SPLIT ? R1 : STAGE];   // stage of even steps
  __shared__ __attribute__((aligned(1024))) unsigned char stB[SPLIT ? R1 : STAGE];   // stage of odd steps
  // the R1 region of a stage
  auto r1 = [&](const unsigned char* st) __attribute__((always_inline)) -> unsigned char* {
    if constexpr (SPLIT) return stB;
    else return const_cast<unsigned char*>(st) + R1;
  };
  extern __shared__ int16_t slist[];         // the row's FULL, LOW (and SKIM) key blocks (list_cap entries)
  __shared__ uint64_t smask[64];             // per visited chunk: bit j = block 64c + j skipped
  __shared__ unsigned char schunk[64];       // chunks holding at least one skipped block
  __shared__ int snc;

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

  const unsigned char* ws = a.ws;
  const int* counts = reinterpret_cast<const int*>(ws + a.L.counts) + row * 4;
  // the list in LDS holds a.list_cap entries, the plan's bound on a row's kept
  // tiles; a row past it (not possible for a valid plan) is cut, never read past
  const int cap = a.list_cap;
  const int nF = min(counts[0], cap), nL = min(counts[1], cap - nF);
  const int nK = nF + nL;
  const int nSk = SKIM ? min(dm.Nk - counts[0] - counts[1] - counts[2], cap - nK) : 0;   // SKIM follows LOW
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
  const int nSteps = sF + 2 * snc + sL + nSk;

  const uint16_t* kin = a.k + toff;
  const unsigned char* slab = ws + a.L.slab + (int64_t)bh * a.L.sl.bytes;
  const Slab SL = a.L.sl;
  // sk is read through the constant address space: a uniform load there is a
  // scalar load, counted by lgkmcnt, so waiting for it does not also wait for
  // the DMA already in flight (a vector load would share vmcnt with it).
  typedef __attribute__((address_space(4))) const float cfloat;
  cfloat* skp = (cfloat*)(reinterpret_cast<const float*>(ws + a.L.sk) + (int64_t)bh * dm.Nk);

  // ---- Q rows of this wave as bf16 B operands: lane (ln, lh) holds
  // q[row][16c + 8lh .. +8] for chunk c.
  const int qrow = I * (32 * NW) + wave * 32 + ln;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; c++) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qrow < dm.N) v = *reinterpret_cast<const uint4*>(a.q + toff + (int64_t)qrow * dm.sn + 16 * c + 8 * lh);
    qreg[c] = __builtin_bit_cast(bf16x8, v);
  }
  const float sq = reinterpret_cast<const float*>(ws + a.L.sq)[row];
  const float cF = kLog2e / __builtin_sqrtf(static_cast<float>(D));

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
    return t < tLow ? G * (t - nS2) + g : (SKIM && t >= tSk) ? nK + (t - tSk) + g : nF + G * (t - tLow) + g;
  };
  auto list_end = [&](int t) { return t < tLow ? nF : nK; };
  auto list_at = [&](int t) { return (int)slist[list_idx(t, 0)]; };

  // ---- DMA of step t's operands into stage `st`.  Region layouts (bytes):
  //   FULL    R0 = K [64][D] bf16,       R1 = V^T [D][64] fp16
  //   LOW     R0 = K8 [64][D] E4M3,      R1 = V low^T [D][64] fp16
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
  // one resource over this head's slab; every workspace operand is a scalar
  // sub-offset of it
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(slab, (uint32_t)SL.bytes);
  // 16-key blocks: LDS slot (row d, chunk lane & 7) of a [D][64] 16-bit tile
  // holds logical chunk lc = (lane & 7) ^ swz128(d), i.e. 8 keys of column
  // group lc / 2; the lane fetches them from that group's block, stored
  // [D][16] (32 bytes per row d), half lc & 1 of the row.
  const int vlc = (lane & 7) ^ ((lane >> 3) & 7) ^ (wave & 1);
  const int vgrp = vlc >> 1;
  const int vlane = (lane >> 3) * 32 + (vlc & 1) * 16;
  // caller's K as one resource per head for 16- and 8-key gathers: rows past N read as zero
  const __amdgpu_buffer_rsrc_t rKh = make_rsrc(kin, (uint32_t)dm.N * (uint32_t)dm.sn * 2);
  // V^T rows of the step's G blocks (per-block [D][BK] layout) from `base`.
  // 16-key blocks: logical chunk vlc holds 8 keys of column group vlc / 2, half
  // vlc & 1 of that block's 32-byte row; 8-key blocks: chunk vlc is slot vlc's
  // whole 16-byte row.
  // jv (8-key blocks): lane g < 8 holds the step's block of slot g
  auto load_vt16g = [&](unsigned char* reg, int base, int jv) __attribute__((always_inline)) {
    if constexpr (G == 1) {
      (void)reg; (void)base; (void)jv;
    } else {
      constexpr int ROWB = BK * 2;                  // bytes per stored V^T row of a block
      const int vo = G == 4 ? vlane + __shfl(jv, vgrp, 64) * (D * ROWB)
                            : (lane >> 3) * ROWB + __shfl(jv, vlc, 64) * (D * ROWB);
#pragma unroll
      for (int i = 0; i < NI16; i++) {
        const int k = wave + NW * i;
        dma16(rS, reg + k * 1024, vo, base + k * 8 * ROWB);
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
  // KINDS: bit mask of the step kinds that can occur where this is called; the
  // other branches are not generated, so their address terms are not kept live.
  // PART: 1 = the R0 half (K, E4M3 K, MXFP4 K and its scales, kbar hi) and
  // the step's score scale; 2 = the R1 half (V^T, low-tier or SKIM V^T, kbar
  // lo, vbar^T); 3 = both.  Per wave, every R1 half is NI16 instructions.
  auto issue_part = [&](auto kinds, auto part, int t, unsigned char* st, StepScale<G>& cst) __attribute__((always_inline)) {
    constexpr int KINDS = decltype(kinds)::value;
    constexpr bool PA = decltype(part)::value & 1, PB = decltype(part)::value & 2;
    const int kind = step_kind(t);
    if constexpr (G > 1) {
      if (((KINDS & (1 << kFull)) && kind == kFull) || ((KINDS & (1 << kLow)) && kind == kLow)) {
        // one block index per lane (lane g < G: the step's g-th block), read
        // straight from the list; a runtime slot then selects by lane, never by
        // indexing an array (which the compiler would place in scratch memory)
        int jv;
        {
          const int i0 = list_idx(t, 0), e = list_end(t), g = lane & (G - 1);
          jv = (int)slist[i0 + g < e ? i0 + g : i0];
        }
        if (kind == kFull) {
          if constexpr (PA) {
#pragma unroll
            for (int i = 0; i < NI16; i++) {
              const int k = wave + NW * i;
              const int row0 = k * RPI;                // first stage row of the instruction
              if constexpr (G == 4) {
                const int Jg = __builtin_amdgcn_readlane(jv, row0 >> 4);
                dma16(rKh, st + k * 1024, lk[i % NSW] + (Jg * 16 + (row0 & 15)) * (int)dm.sn * 2, 0);
              } else if constexpr (D == 128) {
                // score row m = row0 + rr16 takes key kk8(m) of slot slot8(m); an
                // instruction's four rows share one slot
                const int Js = __builtin_amdgcn_readlane(jv, slot8(row0));
                dma16(rKh, st + k * 1024, lk[i % NSW] + (Js * 8 + kk8(row0)) * (int)dm.sn * 2, 0);
              } else {
                const int m = row0 + rr16;
                dma16(rKh, st + k * 1024,
                      lk[i % NSW] + (__shfl(jv, slot8(m), 64) * 8 + kk8(m) - rr16) * (int)dm.sn * 2, 0);
              }
            }
          }
          if constexpr (PB) load_vt16g(r1(st), (int)SL.vt, jv);
          if constexpr (PA) {
#pragma unroll
            for (int g = 0; g < StepScale<G>::N; g++) cst.c[g] = cF;
          }
        } else {
          if constexpr (PA) {
#pragma unroll
            for (int i = 0; i < NI8; i++) {
              const int k = wave + NW * i;
              const int row0 = k * (1024 / D);         // E4M3 rows are D bytes
              if constexpr (G == 4) {
                const int Jg = __builtin_amdgcn_readlane(jv, row0 >> 4);
                dma16(rS, st + k * 1024, voffK8, (int)SL.k8 + (Jg * 16 + (row0 & 15)) * D);
              } else {
                const int ri = D == 128 ? lane >> 3 : lane >> 2;   // row of the lane inside the instruction
                const int m = row0 + ri;
                dma16(rS, st + k * 1024, voffK8 + (__shfl(jv, slot8(m), 64) * 8 + kk8(m) - ri) * D, (int)SL.k8);
              }
            }
          }
          if constexpr (PB) load_vt16g(r1(st), (int)SL.vlow, jv);
          if constexpr (PA) {
#pragma unroll
            for (int g = 0; g < StepScale<G>::N; g++) {
              if constexpr (G == 8) {
                const float s0 = skp[__builtin_amdgcn_readlane(jv, 2 * g)];
                const float s1 = skp[__builtin_amdgcn_readlane(jv, 2 * g + 1)];
                cst.c[g] = sq * (lh ? s1 : s0) * cF;
              } else {
                cst.c[g] = sq * skp[__builtin_amdgcn_readlane(jv, g)] * cF;
              }
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
      if constexpr (PB) load_vt16(r1(st), rS, (int)SL.vt + J * 128 * D);
      if constexpr (PA) cst.c[0] = cF;
    } else if (G == 1 && (KINDS & (1 << kLow)) && kind == kLow) {
      const int J = list_at(t);
      if constexpr (PA) {
#pragma unroll
        for (int i = 0; i < NI8; i++) {
          const int k = wave + NW * i;
          dma16(rS, st + k * 1024, voffK8, (int)SL.k8 + J * 64 * D + k * 1024);
        }
      }
      if constexpr (PB) load_vt16(r1(st), rS, (int)SL.vlow + J * 128 * D);
      if constexpr (PA) cst.c[0] = sq * skp[J] * cF;
    } else if (SKIM && (KINDS & (1 << kSkim)) && kind == kSkim) {
      // MXFP4 K [64][D/2] into R0, its scale bytes [64][D/32] after it (one
      // D/32-byte load per lane from wave 0, into a 4-byte LDS slot per
      // lane), fp16 dequantised V^T into R1
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
      if constexpr (PB) load_vt16(r1(st), rS, (int)SL.vskim + J * 128 * D);
      if constexpr (PA) cst.c[0] = cF;
    } else {
      const int c = schunk[t >> 1];
      if ((KINDS & (1 << kSkipS)) && kind == kSkipS) {
#pragma unroll
        for (int i = 0; i < NI16; i++) {
          const int k = wave + NW * i;
          if constexpr (PA) dma16(rS, st + k * 1024, lkb[i % NSW], (int)SL.kbhi + c * 128 * D + k * 1024);
          if constexpr (PB) dma16(rS, r1(st) + k * 1024, lkb[i % NSW], (int)SL.kblo + c * 128 * D + k * 1024);
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
  int offk[D / 16], offv[4], offk8[D / 32];
#pragma unroll
  for (int c = 0; c < D / 16; c++) offk[c] = offK<D>(ln, 2 * c + lh);
#pragma unroll
  for (int c = 0; c < 4; c++) offv[c] = offV(ln, 2 * c + lh);   // within R1
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
    opaque_arr(lk);
    opaque_arr(lkb);
    opaque(voffV, voffK8);
  };

  // ---- online-softmax state
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; db++) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  f16x8 pb[4];

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
  // S^T of a SKIM step on the block-scaled fp4 MFMA: lane (ln, lh) holds
  // channels 64i + 32lh .. +31 of key rows ln and ln + 32 (from the stage) and
  // of its query row (q4, made once per row): one E8M0 block each, whose
  // scale bytes the MFMA applies (opsel picks the byte of the key row's word).
  auto scores_fp4 = [&](const unsigned char* st, f32x16* s, const i32x8* q4, const int* q4s) __attribute__((always_inline)) {
    const int sw = D == 128 ? (ln >> 2) & 3 : (ln >> 3) & 1;
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
  // score scale of this lane's P chunk cc: one per step (64-key blocks), per
  // 16-key group (16-key blocks), per slot 2 cc + lane half (8-key blocks)
  auto chunk_scale = [&](const StepScale<G>& cs, int cc) __attribute__((always_inline)) {
    if constexpr (G == 1) return cs.c[0];
    else return cs.c[cc];
  };
  auto softmax = [&](f32x16* s, const StepScale<G>& cs, float tmax) __attribute__((always_inline)) {
    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool need = tmax > m_run + kLazy;
    if (__ballot(need)) {
      const float mn = need ? tmax : m_run;
      const float al = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
      l_run *= al;
#pragma unroll
      for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[db][r] *= al;
      m_run = mn;
    }
    const float nm = -m_run;
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int tt = 0; tt < 8; tt++) {
        const int e = 8 * cc + tt;
        pb[cc][tt] = static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 4][e & 15], chunk_scale(cs, cc), nm)));
      }
    // l accumulates the fp16 P values the P.V MFMA multiplies, two per
    // v_dot2_f32_f16 (fp32 accumulation)
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    float psum = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
#pragma unroll
      for (int j = 0; j < 4; j++) psum = __builtin_amdgcn_fdot2(h2{pb[cc][2 * j], pb[cc][2 * j + 1]}, one2, psum, false);
    l_run += psum;
  };
  auto row_max = [&](const f32x16* s) __attribute__((always_inline)) {
    float m = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) m = __builtin_fmaxf(m, s[b][r]);
    return m;
  };
  // ---- O^T += V^T P^T from region R1 (fp16 V, low-tier V, or block means)
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
  // a kept tile (FULL: bf16 scores, LOW: E4M3 scores): masks and softmax of
  // its scores s
  auto kept_soft = [&](auto low_tag, int t, f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) {
    constexpr bool LOW = decltype(low_tag)::value;
    if constexpr (G == 1) {
      const int J = list_at(t);
      if (J == dm.Nk - 1) mask_tail(s, dm.N - 64 * J);
      softmax(s, c, row_max(s) * c.c[0]);
    } else {
      // Lists are ascending, so a partial group or the ragged last block only
      // occurs in the last step of the phase.  Register (b, r) is key
      // 8((r >> 2) & 1) + 4lh + r % 4 of 16-key block 2b + r / 8, or key
      // 4((r >> 2) & 1) + r % 4 of 8-key block (slot) 4b + 2(r / 8) + lh.
      if (t == (LOW ? tSk - 1 : tLow - 1)) {
        const int i0 = list_idx(t, 0), e = list_end(t);
        // valid keys of each block: 0 past the list end, fewer in block Nk - 1
        int lim[G];
#pragma unroll
        for (int g = 0; g < G; g++) {
          const int Jg = (int)slist[i0 + g < e ? i0 + g : i0];
          lim[g] = i0 + g >= e ? 0 : Jg == dm.Nk - 1 ? dm.N - BK * Jg : BK;
        }
        // this lane's limit for P chunk q = 2b + (r >> 3), against the key index
        // of register r inside its block
        int ql[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          ql[q] = G == 4 ? lim[q] - 4 * lh : (lh ? lim[2 * q + 1] : lim[2 * q]);
          opaque(ql[q]);
        }
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int kk = G == 4 ? 8 * ((r >> 2) & 1) + (r & 3) : (r & 3) + 4 * ((r >> 2) & 1);
            if (kk >= ql[2 * b + (r >> 3)]) s[b][r] = -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int cc = 0; cc < 4; cc++) {
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < 8; r++) m = __builtin_fmaxf(m, s[cc >> 1][8 * (cc & 1) + r]);
        tmax = __builtin_fmaxf(tmax, m * chunk_scale(c, cc));
      }
      softmax(s, c, tmax);
    }
  };
  // a kept tile staged in `st`: scores, softmax, P.V
  auto kept_step = [&](auto low_tag, int t, const unsigned char* st, const StepScale<G>& c, const i32x8* q8) __attribute__((always_inline)) {
    f32x16 s[2] = {f32x16{}, f32x16{}};
    if constexpr (decltype(low_tag)::value) scores_fp8(st, s, q8);
    else scores_bf16(st, s);
    kept_soft(low_tag, t, s, c);
    pv(st);
  };
  // a SKIM tile (64-key blocks): mask and softmax of its scores s
  auto skim_soft = [&](int t, f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) {
    const int J = list_at(t);
    if (J == dm.Nk - 1) mask_tail(s, dm.N - 64 * J);
    softmax(s, c, row_max(s) * c.c[0]);
  };
  auto skim_step = [&](int t, const unsigned char* st, const StepScale<G>& c, const i32x8* q4, const int* q4s) __attribute__((always_inline)) {
    f32x16 s[2] = {f32x16{}, f32x16{}};
    scores_fp4(st, s, q4, q4s);
    skim_soft(t, s, c);
    pv(st);
  };
  // pooled keys of a chunk of 64 skipped-candidate blocks: scores only (hi
  // part from R0, lo part from R1), then the bias and the softmax
  auto skip_S = [&](const unsigned char* st, f32x16* s) __attribute__((always_inline)) {
    scores_bf16(st, s);
    scores_bf16(r1(st), s);   // low half of kbar
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
    constexpr float lgfull = BK == 64 ? 6.0f : BK == 16 ? 4.0f : 3.0f;   // log2(BK)
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
    softmax(s, one, tmax);
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
  };
  // the MXFP4 copy of this lane's Q row (channels 64i + 32lh .. +31 for
  // instruction i, one E8M0 scale each), from Q in memory
  auto make_q4 = [&](i32x8* q4reg, int* q4s) __attribute__((always_inline)) {
    const uint16_t* qp = a.q + toff + (int64_t)qrow * dm.sn + 32 * lh;
#pragma unroll
    for (int i = 0; i < D / 64; i++) {
      float x[32];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (qrow < dm.N) raw = *reinterpret_cast<const uint4*>(qp + 64 * i + 8 * j);
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const float f = __uint_as_float(e & 1 ? (wd[e >> 1] & 0xffff0000u) : (wd[e >> 1] << 16));
          x[8 * j + e] = f;
          amax = __builtin_fmaxf(amax, __builtin_fabsf(f));
        }
      }
      const int ex = mx4_exponent(amax);
      uint32_t pk[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 32; e++) pk[e >> 3] |= e2m1_code(ldexpf(x[e], -ex)) << (4 * (e & 7));
      q4reg[i] = i32x8{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], 0, 0, 0, 0};
      q4s[i] = ex + 127;
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
                     // fp8 instruction i = bf16 chunks 4i..4i+3)
      i32x8 q8reg[D / 64];
      make_q8(q8reg);
      run_phase(tSk, [&](auto p, int tt) __attribute__((always_inline)) {
        if (tt + 1 < nSteps) issue(KLow{}, tt + 1, stg(flip(p)), scl(flip(p)));
        kept_step(std::true_type{}, tt, stg(p), scl(p), q8reg);
        next();
      });
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
      if (k == kLow) return NI8;
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
    // read R1 (a skip chunk's lo half).
    auto split_step = [&](auto nk, auto hs, auto hp, auto u1, auto S_fn, auto soft_fn) __attribute__((always_inline)) {
      constexpr bool HS = decltype(hs)::value, HP = decltype(hp)::value, U1 = decltype(u1)::value;
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
        pv(stA);
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
        split_step(KSkipPV{}, T1{}, T0{}, T1{},
                   [&](f32x16* s) __attribute__((always_inline)) { skip_S(stA, s); },
                   [&](f32x16* s, const StepScale<G>&) __attribute__((always_inline)) { skip_soft(t, s); });
      else
        split_step(KAfterSkip{}, T0{}, T1{}, T0{}, no_S, no_soft);
    }
    while (t < tLow)
      split_step(KAfterFull{}, T1{}, T1{}, T0{},
                 [&](f32x16* s) __attribute__((always_inline)) { scores_bf16(stA, s); },
                 [&](f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) { kept_soft(T0{}, t, s, c); });
    if (t < tSk) {
      i32x8 q8reg[D / 64];
      make_q8(q8reg);
      while (t < tSk)
        split_step(KLow{}, T1{}, T1{}, T0{},
                   [&](f32x16* s) __attribute__((always_inline)) { scores_fp8(stA, s, q8reg); },
                   [&](f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) { kept_soft(T1{}, t, s, c); });
    }
    if constexpr (SKIM) {
      if (t < nSteps) {
        i32x8 q4reg[D / 64];
        int q4s[D / 64];
        make_q4(q4reg, q4s);
        while (t < nSteps)
          split_step(KSkimOnly{}, T1{}, T1{}, T0{},
                     [&](f32x16* s) __attribute__((always_inline)) { scores_fp4(stA, s, q4reg, q4s); },
                     [&](f32x16* s, const StepScale<G>& c) __attribute__((always_inline)) { skim_soft(t, s, c); });
      }
    }
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
  if (a.skim && a.d.Bk != 64) return hipErrorInvalidValue;
  if (a.d.Nk > kMaxNk || a.list_cap < 1 || a.list_cap > a.d.Nk) return hipErrorInvalidValue;
  const size_t lds = ((size_t)a.list_cap * 2 + 15) / 16 * 16;   // the row's list (dynamic LDS)
  const dim3 grid(a.d.BH * a.d.Nq), block(NW * 64);
  if (a.skim)
    hipLaunchKernelGGL((k3_attn<D, NW, 64, true>), grid, block, lds, s, a);
  else if (a.d.Bk == 64)
    hipLaunchKernelGGL((k3_attn<D, NW, 64, false>), grid, block, lds, s, a);
  else if (a.d.Bk == 16)
    hipLaunchKernelGGL((k3_attn<D, NW, 16, false>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((k3_attn<D, NW, 8, false>), grid, block, lds, s, a);
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
