/*
 * tattn.h -- three-tier tile-sparse attention for AMD Instinct MI355X (gfx950).
 *
 * The library computes, per (batch, head), an approximation of
 * softmax(Q K^T / sqrt(d)) V in which every (query-block I, key-block J) tile
 * runs in one of three tiers:
 *   FULL  exact scores and values in bf16 (fp32 accumulation),
 *   LOW   fp8 E4M3 operands with one scale per block,
 *   SKIP  the tile is replaced by its block means: one score
 *         q_i . kbar_J / sqrt(d) + ln n_J valued by vbar_J,
 * and optionally a fourth, between LOW and SKIP:
 *   SKIM  MXFP4 operands (E2M1 codes, one power-of-two E8M0 scale per 32
 *         channels of a token row) on the block-scaled fp4 MFMA.
 * Tiers come from a block router, p_IJ = softmax_J(qbar_I . kbar_J / sqrt(d)
 * + ln n_J), with dual thresholds tau_hi / tau_lo and an optional per-row
 * top-k, or from an entropy-derived per-head top-k, or from a per-tile error
 * prediction weighed against one price; diagonal tiles are always FULL.
 * Sources of the method:
 *   - "Triage" (abstract): three approximation tiers per tile, skipping by
 *     block means, skimming in a 4-bit floating-point format (the SKIM tier
 *     here), one fused kernel over all tiers in a single pass; a
 *     router that predicts each tile's error under each tier from block
 *     statistics and promotes a tile only when the error reduction pays for
 *     the extra compute at a single price.
 *   - "APT" (abstract): attention probability as the importance metric; dual
 *     thresholds select elements and assign precision; mask management and
 *     tile dataflow.
 *   - "HierPAS" (abstract): a lightweight eager estimate of the attention
 *     pattern, sampling-based entropy for head-wise retention ratios,
 *     progressively reduced precision, a top-k engine.
 *   - "FG-Attn" (abstract): M x N tile granularity (key blocks of 64, 16, 8,
 *     4, 2 or 1 keys here; blocks below 64 keys are gathered 64 / block_k at
 *     a time into dense 64-key MFMA slabs).
 *
 * Conventions
 *   - Every pointer is a DEVICE pointer unless its comment says "host".
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Calls are asynchronous on `stream` except those marked SYNC, which
 *     synchronise `stream` before returning.
 *   - Every call returns a tattn_status; nothing aborts and no C++ exception
 *     crosses the ABI.  tattn_last_error() gives a thread-local message for
 *     the last failing call on the calling thread.
 *   - Arguments are validated before anything is launched: a call that
 *     returns an error has launched nothing and written nothing.
 *   - Tensors Q, K, V, O are [batch, heads, seq_len, head_dim] bf16 (O may
 *     be fp32), head_dim contiguous, sharing the element strides of the
 *     config; base pointers 16-byte aligned and stride_n a multiple of 8.
 *   - The library never allocates device memory: the caller passes a
 *     workspace of tattn_workspace_bytes() bytes and owns it.
 */
#ifndef TATTN_H
#define TATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TATTN_OK = 0,
  TATTN_E_INVALID = -1,      /* a null pointer, bad size, bad threshold, misalignment */
  TATTN_E_UNSUPPORTED = -2,  /* a valid request outside what the kernels implement    */
  TATTN_E_WORKSPACE = -3,    /* workspace missing, misaligned or too small             */
  TATTN_E_HIP = -4,          /* a HIP runtime call or kernel launch failed             */
  TATTN_E_STATE = -5         /* a plan used against other tensors, or in the wrong mode */
} tattn_status;

/* Tier-map byte values.  By accuracy: FULL > LOW > SKIM > SKIP. */
typedef enum { TATTN_SKIP = 0, TATTN_LOW = 1, TATTN_FULL = 2, TATTN_SKIM = 3 } tattn_tier;

typedef enum {
  TATTN_MODE_THRESHOLD = 0,  /* FULL if p >= tau_hi, LOW if tau_lo <= p < tau_hi, else SKIP,
                                except SKIM if tau_skim > 0 and tau_skim <= p < tau_lo;
                                top_k > 0 first keeps only the row's top_k tiles        */
  TATTN_MODE_ADAPTIVE = 1,   /* per head k_h from the entropy of p on sampled rows; per row
                                the top ceil(full_frac*k_h) tiles FULL, the rest of the top
                                k_h LOW, the remainder SKIP (SKIM where tau_skim > 0 and
                                p >= tau_skim)                                           */
  TATTN_MODE_ALL_FULL = 2,   /* every tile FULL: dense attention through the same kernel */
  TATTN_MODE_EXTERNAL = 3,   /* tiers supplied with tattn_plan_set_tiers                 */
  TATTN_MODE_PRICE = 4       /* each tile takes the tier minimising predicted error plus
                                price * work, the error predicted from block second
                                moments (see tattn_plan)                                 */
} tattn_mode;

typedef enum { TATTN_BF16 = 0, TATTN_FP32 = 1 } tattn_dtype;

typedef struct {
  int32_t batch, heads, seq_len, head_dim; /* head_dim in {64, 128}                          */
  int32_t block_q, block_k;                /* block_q 64 or 128; block_k 64, 16, 8, 4, 2, 1  */
  float tau_hi, tau_lo;                    /* 0 <= tau_lo <= tau_hi, finite                  */
  int32_t top_k;                           /* 0 = off, else 1..ceil(seq_len/block_k)         */
  int32_t mode;                            /* tattn_mode                                     */
  float keep_min, keep_max, full_frac;     /* ADAPTIVE: retention clip and FULL share        */
  int32_t entropy_samples;                 /* ADAPTIVE: number of sampled query blocks       */
  int32_t in_dtype, out_dtype;             /* in: TATTN_BF16; out: TATTN_BF16 or TATTN_FP32  */
  int64_t stride_b, stride_h, stride_n;    /* element strides shared by Q, K, V and O        */
  float price;                             /* PRICE: error per FULL tile of work, >= 0,
                                              finite; ignored by the other modes             */
  float tau_skim;                          /* 0 = no SKIM tier.  > 0 (finite) enables it:
                                              THRESHOLD uses it as the SKIM / SKIP
                                              threshold (then <= tau_lo), ADAPTIVE makes a
                                              tile outside the kept ones SKIM where p >=
                                              tau_skim, EXTERNAL accepts SKIM bytes, PRICE
                                              weighs SKIM as a fourth choice; ignored by
                                              ALL_FULL                                       */
  int32_t low_refine;                      /* 0: LOW tiles score on E4M3 copies of Q and K.
                                              1 (no SKIM tier): they score on
                                              MXFP4 copies with an MXFP4 residual correction
                                              ("Triage": refining a tile with 4-bit residual
                                              correction): <q4,k4> + <q4,k4r> + <q4r,k4>;
                                              probabilities and values as before          */
} tattn_config;

typedef struct tattn_plan_s* tattn_plan_t;  /* opaque host object; device state is in the workspace */

typedef struct {
  int64_t n_full, n_low, n_skip;  /* tiles per tier, over all (b, h, I, J)           */
  int64_t n_diag;                 /* diagonal tiles (always FULL)                    */
  double flops_bf16;              /* 16-bit MFMA flops: FULL tiles (4 m n d), SKIP
                                     tiles (4 m d: one pooled key each), and the
                                     P.V half of LOW and SKIM tiles with blocks
                                     below 64 keys                                  */
  double flops_fp8;               /* fp8 MFMA flops: LOW tiles (4 m n d with 64-key
                                     blocks, else the score half), the P.V half of
                                     SKIM tiles with 64-key blocks                  */
  double flops_dense;             /* 4 * N^2 * d * B * H: dense-equivalent work      */
  int64_t n_skim;                 /* SKIM tiles                                      */
  double flops_fp4;               /* fp4 MFMA flops: the score half of SKIM tiles,
                                     and of refined LOW tiles (three fp4 passes)    */
} tattn_stats;

/* Check a config without touching any device.  Host only; no HIP calls. */
tattn_status tattn_validate(const tattn_config* cfg);

/* Bytes of workspace that tattn_plan needs for `cfg` (host only).  The
 * workspace must be 256-byte aligned; its layout is private to the library. */
tattn_status tattn_workspace_bytes(const tattn_config* cfg, size_t* bytes /* host out */);

/*
 * Build a plan: block pooling, fp8 quantisation and routing.
 *  1. Block means qbar_I, kbar_J, vbar_J (float64 sums, stored as float32) and,
 *     per block, amax, scale = amax/448 and E4M3 codes of K and V, plus the
 *     Q-block scales ("Triage": block means; "HierPAS": reduced precision).
 *  2. Router p_IJ = softmax_J(qbar_I . kbar_J / sqrt(d) + ln n_J) in float64
 *     ("APT": attention probability as importance), and
 *  3. the tier map by `cfg->mode` (dual thresholds, top-k, entropy-adaptive,
 *     all-full, price) with diagonal tiles forced FULL, compacted per query
 *     block into [FULL asc | LOW asc | SKIP asc] key-block lists.
 * TATTN_MODE_PRICE ("Triage": error predicted from block statistics, one
 * price) also takes second moments in step 1 (per block and dimension the
 * mean square of Q and the variance of K; per key block the variance total,
 * mean-square total and mean norm of V and the mean-square total of K).  Per
 * tile it predicts the within-tile score spread
 * s2 = sum_c q2[I,c] kvar[J,c] / d, a lognormal log-mass gain g (s2/2, or
 * sqrt(2 s2 ln n_J) - ln n_J beyond s2 = 2 ln n_J) and n_eff =
 * max(1, n_J e^-s2); the relative errors
 *   SKIP  vnorm (1 - e^-g) + sqrt(vvar max(0, 1/n_eff - 1/n_J)),
 *   LOW   vnorm expm1(sl2/2) + (sqrt(vvar expm1(sl2)) + u sqrt(m2v/3)) / sqrt(n_eff),
 *         sl2 = (2u^2/3) m2q m2k / d^2, u = 2^-4,
 *   FULL  0;
 *   SKIM  (with tau_skim > 0) the LOW form with u = 2^-2 (MXFP4);
 * shares p~ = softmax_J(S + g); and gives the tile the tier with the least
 * p~ * error + price * work (work FULL 1, LOW 0.75, SKIM 0.625, SKIP
 * 1.5 / block_k; ties to the cheaper tier).  All in float64.
 * q, k, v: the caller's tensors.  The plan keeps derived copies of K and V
 * (E4M3 and MXFP4 codes, the low tier's dequantised V for blocks below 64
 * keys, means) in `workspace`, and FULL tiles read k and v themselves, so a
 * later tattn_forward must be given the same k and v pointers with unchanged
 * contents.  *out receives a new host handle (free with tattn_plan_destroy);
 * it stays valid while the workspace lives.  In TATTN_MODE_EXTERNAL the
 * router is not run and the plan has no tiers until tattn_plan_set_tiers.
 */
tattn_status tattn_plan(const tattn_config* cfg, const void* q, const void* k, const void* v,
                        void* workspace, size_t workspace_bytes, void* stream, tattn_plan_t* out);

/*
 * The fused three-tier pass ("Triage": one kernel, all tiers, single pass):
 * for every query block, an online softmax over its FULL tiles (bf16 MFMA),
 * its LOW tiles, its SKIM tiles and its SKIP tiles (block means with a ln n_J
 * bias), then O = acc / l.  A LOW tile's scores come from E4M3 Q and K on the
 * fp8 MFMA ("HierPAS": reduced precision for less critical tiles; "APT":
 * dual-precision execution); its probabilities are quantised to E4M3 against
 * the tile's row maximum (x_j = 448 e^{s_j - m_t}, so the maximum is 448), and
 * P.V runs on the fp8 MFMA against the E4M3 V (64-key blocks; with smaller
 * blocks the quantised probabilities meet the dequantised V in fp16),
 * the row normaliser summing the same quantised probabilities.  A SKIM tile
 * ("Triage": skimming in 4 bits) takes its scores from MXFP4 Q and K on the
 * block-scaled fp4 MFMA and is otherwise a LOW tile.
 * q: the queries; the LOW tier's per-block Q scales are taken from q itself,
 * so q may differ from the tensor the plan was routed with (the tiers stay
 * the plan's).  o: output tensor with the config's strides, dtype
 * cfg->out_dtype.  k and v must be the pointers the plan was built with
 * (TATTN_E_STATE if not).
 */
tattn_status tattn_forward(tattn_plan_t plan, const void* q, const void* k, const void* v, void* o,
                           void* stream);

/*
 * tattn_forward that also writes the probability codes of the LOW and SKIM
 * steps of selected query blocks, for checking them against a reference
 * (several codes are correct where 448 e^{s - m_t} lies on a rounding
 * midpoint to within the precision of the scores).  Same arithmetic and
 * output as tattn_forward.
 *   dump_slot  device int32 [B*H*Nq]: slot of query block (b, h, I) at index
 *              (b*H + h)*Nq + I, or -1 for a block not dumped
 *   dump_steps device-side stride in steps per slot; a row's LOW steps come
 *              first, then its SKIM steps, and steps >= dump_steps are not
 *              written
 *   dump       device uint8 [slots][dump_steps][block_q][64], 16-byte aligned:
 *              byte (slot, step s, query row i of the block, 32 h + p) is the
 *              code of score register (b = p / 16, r = p % 16) of lane half h,
 *              i.e. of staged key 32 b + 8 (r / 4) + 4 h + r % 4 of the step.
 *              A 64-key step is one key block; a 16-key step gathers the next
 *              four list entries (staged key m: block m / 16, key m % 16); a
 *              step of BK <= 8 keys per block gathers 64 / BK (staged key m:
 *              block p / BK, key p % BK of the step's blocks, p = m with bits
 *              2 and 3 swapped).  Codes of keys past a block's end are 0; with
 *              one-key blocks every live key's code is 448 (0x7E).  Unwritten
 *              bytes keep their contents.
 * TATTN_E_INVALID for NULL pointers or dump_steps < 1; otherwise as
 * tattn_forward.
 */
tattn_status tattn_forward_dump(tattn_plan_t plan, const void* q, const void* k, const void* v, void* o,
                                const int32_t* dump_slot, int32_t dump_steps, uint8_t* dump, void* stream);

/*
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): tattn_plan followed
 * by tattn_forward in one call, with the workspace in a static device array
 * of the library (64 MiB on each GPU the library runs on, held until the
 * process ends) instead of the caller's.  Calls no allocating routine.
 * cfg: any routed mode (EXTERNAL gives TATTN_E_STATE); q, k, v, o as for
 * tattn_plan / tattn_forward.  TATTN_E_WORKSPACE, before anything is
 * launched, when tattn_workspace_bytes(cfg) exceeds 64 MiB.  Every call on a
 * GPU uses that GPU's one array: calls that overlap on one GPU (two streams,
 * two threads) race and give undefined results; calls in one stream are
 * ordered.  The array keeps the last call's contents; every region a call
 * reads it has written first.  Asynchronous on `stream`.
 */
tattn_status tattn_attention_static(const tattn_config* cfg, const void* q, const void* k, const void* v, void* o,
                                    void* stream);

/* Host only.  The most kept (FULL, LOW or SKIM) tiles a query block can hold
 * under `cfg`'s tier rule, which sizes the fused kernel's per-row list: the
 * top k_h bound ceil(keep_max * Nk) plus the diagonal blocks (ADAPTIVE), top_k
 * plus the diagonal blocks (THRESHOLD with top-k), else Nk.  A forward that
 * meets a row above it cuts the row and flags the plan; tattn_plan_stats then
 * returns TATTN_E_STATE. */
tattn_status tattn_list_bound(const tattn_config* cfg, int32_t* bound /* host out */);

/*
 * Reuse a plan for the next diffusion step ("APT": attention probabilities
 * predicted across timesteps from their temporal similarity): the tier map,
 * lists and work order stay those of the step the plan was routed on, and
 * step 1 of tattn_plan (block means, scales, E4M3 codes, the transposed V
 * copies, and in PRICE mode the second moments) is recomputed
 * from q, k, v, the next step's tensors, which must have the config's shape
 * and strides.  The router is not run.  Afterwards the plan belongs to these
 * k and v (tattn_forward checks the pointers).  Asynchronous on `stream`;
 * TATTN_E_INVALID for a NULL or misaligned pointer, TATTN_E_STATE for a plan
 * that has no tiers yet.
 */
tattn_status tattn_replan(tattn_plan_t plan, const void* q, const void* k, const void* v, void* stream);

/* SYNC.  Replace the plan's tier map with a host map [B, H, Nq, Nk] of bytes in
 * {0, 1, 2}, or {0, 1, 2, 3} when the config has tau_skim > 0; diagonal tiles
 * are forced FULL and the lists rebuilt.  Only for a plan built in
 * TATTN_MODE_EXTERNAL (TATTN_E_STATE otherwise); any other byte gives
 * TATTN_E_INVALID and leaves the plan unchanged. */
tattn_status tattn_plan_set_tiers(tattn_plan_t plan, const uint8_t* host_tiers, void* stream);

/* SYNC.  Copy out the tier map [B, H, Nq, Nk] (bytes) and/or the router
 * probabilities p [B, H, Nq, Nk] (float32, rounded from the float64 values;
 * zero in ALL_FULL and EXTERNAL modes).  Either host pointer may be NULL. */
tattn_status tattn_plan_get_tiers(tattn_plan_t plan, uint8_t* host_tiers, float* host_p, void* stream);

/* SYNC.  Copy out the compacted lists [B, H, Nq, Nk] (int16 key-block indices,
 * per row FULL ascending, then LOW ascending, then SKIM ascending, then SKIP
 * ascending) and/or the counts [B, H, Nq, 3] (int32: n_full, n_low, n_skip;
 * the row's SKIM count is Nk minus their sum).  Either may be NULL. */
tattn_status tattn_plan_get_lists(tattn_plan_t plan, int16_t* host_lists, int32_t* host_counts,
                                  void* stream);

/* SYNC.  Copy out the pooled statistics: qbar [B,H,Nq,d], kbar and vbar
 * [B,H,Nk,d] (float32), and the E4M3 scales sq [B,H,Nq], sk and sv [B,H,Nk]
 * (float32, amax/448, 1 for an all-zero block).  Any pointer may be NULL. */
tattn_status tattn_plan_get_pool(tattn_plan_t plan, float* qbar, float* kbar, float* vbar, float* sq,
                                 float* sk, float* sv, void* stream);

/* SYNC.  Copy out, in the canonical layout [B, H, seq_len, head_dim], the
 * E4M3 codes of K and of V (bytes, E(x * inv) with the block's inverse scale
 * fl32(448 / amax)).  Either may be NULL. */
tattn_status tattn_plan_get_codes(tattn_plan_t plan, uint8_t* host_k8, uint8_t* host_v8, void* stream);

/* SYNC.  SKIM tier (config tau_skim > 0; TATTN_E_STATE otherwise): copy out,
 * in the canonical layout, the MXFP4 copy of K.  k4 [B, H, seq_len,
 * head_dim/2] bytes: E2M1 codes, channel 2m in the low nibble of byte m and
 * 2m+1 in the high nibble; k4s [B, H, seq_len, head_dim/32] bytes: the E8M0
 * scale of each 32 channels, e + 127 for the scale 2^e, e = floor(log2(amax))
 * - 2 clamped to [-127, 127] (-127 for an all-zero block).  Either pointer may
 * be NULL. */
tattn_status tattn_plan_get_mx4(tattn_plan_t plan, uint8_t* host_k4, uint8_t* host_k4s, void* stream);

/* SYNC.  Refined low tier (config low_refine = 1; TATTN_E_STATE otherwise):
 * copy out, in tattn_plan_get_mx4's layouts, the MXFP4 copy of K's rounding
 * residual k - dequant(k4): codes k4r and E8M0 scale bytes k4rs, with the
 * same per-32-channel rule applied to the residual.  tattn_plan_get_mx4 gives
 * the first-level copy under this config too.  Either pointer may be NULL. */
tattn_status tattn_plan_get_mx4_residual(tattn_plan_t plan, uint8_t* host_k4r, uint8_t* host_k4rs, void* stream);

/* SYNC.  PRICE mode: copy out the block second moments the router used
 * (float32): q2 [B,H,Nq,d] and m2q [B,H,Nq] (query mean square per dimension
 * and its total), kvar [B,H,Nk,d] and m2k [B,H,Nk] (key variance per
 * dimension, key mean-square total), vvar, m2v, vnorm [B,H,Nk] (value variance
 * total, mean-square total, norm of the mean).  Each from float64 sums,
 * rounded once.  Any pointer may be NULL; TATTN_E_STATE for other modes. */
tattn_status tattn_plan_get_moments(tattn_plan_t plan, float* q2, float* m2q, float* kvar, float* m2k,
                                    float* vvar, float* m2v, float* vnorm, void* stream);

/* SYNC.  Tier counts and executed / dense-equivalent flops of the plan.
 * TATTN_E_STATE if a forward on this plan cut a row at its list bound (see
 * tattn_list_bound); the flag is cleared by the next tattn_plan or
 * tattn_replan. */
tattn_status tattn_plan_stats(tattn_plan_t plan, tattn_stats* host_out);

/* SYNC.  ADAPTIVE mode: per (b, h) k_h (int32 [B*H]) and r_h (float64 [B*H]);
 * either may be NULL.  TATTN_E_STATE for other modes. */
tattn_status tattn_plan_get_kh(tattn_plan_t plan, int32_t* host_kh, double* host_rh);

/* Free the host handle (the workspace stays the caller's).  NULL is ignored. */
void tattn_plan_destroy(tattn_plan_t plan);

/* Static strings; never NULL. */
const char* tattn_status_str(tattn_status status);
const char* tattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TATTN_H */
