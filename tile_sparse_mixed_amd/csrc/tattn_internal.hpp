// Internal interfaces of the tattn library: workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/tattn.h"

namespace tattn {

constexpr int kTile = 64;          // key-tile width the fused kernel works in
constexpr int kMaxNk = 4096;       // key blocks per row (router and fused-kernel LDS rows)
constexpr int kAlign = 256;

// Sizes derived from a validated config.
struct Dims {
  int B, H, BH, N, D, Bq, Bk, Nq, Nk;
  int NkC;   // chunks of 64 key blocks: ceil(Nk / 64)
  int64_t sb, sh, sn;
};

// Per-head slab of everything the fused kernel reads besides Q and the
// caller's K: one contiguous block per (b, h), so a single buffer resource
// with scalar sub-offsets covers it.  Offsets are bytes from the slab start.
struct Slab {
  size_t v8t;     // u8   [Nk][D][Bk]   E4M3 V^T: 64-key blocks in the fp8 P.V operand's
                  //                    key order (pv8_key), smaller blocks in key order
  size_t vlow;    // fp16 [Nk][Bk][D]   blocks below 64 keys only: the low tier's fp16 V
                  //                    operand fl16(fl32(decode(E4M3) * sv)) as rows
  size_t k8;      // u8   [Nk][Bk][D]   E4M3 K, d permuted within a row (k8_pos)
  size_t kbhi;    // bf16 [Nk][D]       K block means, hi part
  size_t kblo;    // bf16 [Nk][D]       K block means, lo part (kbar = hi + lo to ~2^-17)
  size_t vbarT;   // fp16 [NkC][D][64]  V block means transposed per chunk of 64 blocks,
                  //                    vt_pos order, zero past Nk
  // SKIM tier or refined low tier only (zero-sized otherwise)
  size_t k4;      // u8   [Nk][64][D/2]  MXFP4 K codes, channel 2m in the low nibble of byte m
  size_t k4s;     // u8   [Nk][64][D/32] E8M0 scale of each 32 channels of a K row
  // refined low tier only: the MXFP4 copy of the residual k - dequant(k4)
  size_t k4r;     // u8   [Nk][64][D/2]
  size_t k4rs;    // u8   [Nk][64][D/32]
  size_t bytes;   // slab size (256-byte multiple)
};

// Byte offsets of every region inside the caller's workspace.
struct Layout {
  size_t qbar, kbar, vbar;      // f32 [BH][Nq|Nk][D]
  size_t sq, iq;                // f32 [BH][Nq]   scale and inverse scale of each Q block
  size_t sk, sv;                // f32 [BH][Nk]
  size_t slab;                  // [BH] slabs of Slab::bytes each
  Slab sl;
  size_t S;                     // f64 [BH][Nq][Nk]   router logits (scratch)
  size_t p;                     // f32 [BH][Nq][Nk]
  size_t tiers;                 // u8  [BH][Nq][Nk]
  size_t lists;                 // i16 [BH][Nq][Nk]
  size_t counts;                // i32 [BH][Nq][4]   n_full, n_low, n_skip, fused-kernel steps
                                //                   (n_skim = Nk - n_full - n_low - n_skip)
  size_t order;                 // i32 [BH * Nq]     the fused kernel's row order
  size_t ent;                   // f64 [BH][Ssamp]   entropy of the sampled rows
  size_t kh;                    // i32 [BH]
  size_t rh;                    // f64 [BH]
  // price router only (zero-sized otherwise): block second moments, f32
  size_t q2, m2q;               // [BH][Nq][D], [BH][Nq]   query mean square per dim, total
  size_t kvar, m2k;             // [BH][Nk][D], [BH][Nk]   key variance per dim, mean-square total
  size_t vvar, m2v, vnorm;      // [BH][Nk] each           value variance total, mean-square total, mean norm
  size_t s2;                    // f64 [BH][Nq][Nk]        within-tile score spread
  size_t flag;                  // i32 [4]   device-side error flags (cleared by the pooling
                                //           kernel; [0] bit 0: a row held more kept tiles
                                //           than the fused kernel's list bound)
  size_t total;
};

Dims make_dims(const tattn_config& c);
Layout make_layout(const Dims& d, int entropy_samples, bool moments, bool skim, bool refine);

// ---- launchers (all asynchronous on `s`; return the launch status)
struct PoolArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  unsigned char* ws;
  Layout L;
  Dims d;
  int moments;   // also write the second-moment statistics (price router)
  int mx4;       // also write the MXFP4 copy of K (SKIM tier, refined low tier)
  int resid;     // and the MXFP4 copy of its residual (refined low tier)
};
hipError_t launch_pool(const PoolArgs& a, hipStream_t s);

struct RouterArgs {
  unsigned char* ws;
  Layout L;
  Dims d;
  int mode;
  float tau_hi, tau_lo;
  int top_k;
  float keep_min, keep_max, full_frac;
  int samples;
  float price;
  float tau_skim;   // > 0: THRESHOLD tiles with tau_skim <= p < tau_lo are SKIM
};
hipError_t launch_router(const RouterArgs& a, hipStream_t s);
// Rebuild lists and counts from the tier map already in the workspace
// (diagonal tiles forced FULL first).
hipError_t launch_compact(const RouterArgs& a, hipStream_t s);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;   // FULL tiles read the caller's V rows
  void* o;
  int out_fp32;
  unsigned char* ws;
  Layout L;
  Dims d;
  int skim;       // the plan may hold SKIM tiles (64-key blocks)
  int refine;     // LOW tiles score on MXFP4 with residual correction
  int list_cap;   // bound on a row's FULL + LOW + SKIM tiles under the plan's mode (<= Nk)
  // probability-code dump (tattn_forward_dump; null otherwise): row r with
  // dslot[r] >= 0 writes the codes of its LOW and SKIM steps s < dsteps to
  // dump[((dslot[r] * dsteps + s) * Bq + row in block) * 64 + 32 * half + p]
  const int* dslot;
  unsigned char* dump;
  int dsteps;
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
// the fused pass of one key-block size (k3_bk*.hip)
hipError_t launch_attn_bk64(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bk16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bk8(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bk4(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bk2(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bk1(const AttnArgs& a, hipStream_t s);

}  // namespace tattn
