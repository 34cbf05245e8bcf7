/*
 * bgtq.h -- C ABI of the Block-GTQ packed-KV library for AMD MI355X (gfx950).
 *
 * Block-GTQ ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract)
 * scores every 2-D RoPE frequency block of every (layer, KV head) with a
 * label-free Q/K energy, greedily gives integer bit widths to the blocks by
 * marginal gain under a fixed average budget, encodes keys with TurboQuant-MSE
 * per group of equal-width blocks (values at one uniform width), and serves
 * decode attention straight from the packed cache.  The Block-GTQ README
 * (introduction, calibration paragraph, backend table) adds the per-(layer,
 * KV head) calibration from saved Q/K activations and the fused packed-cache
 * decode kernel as the production path.
 *
 * Conventions (all entry points):
 *  - Return BGTQ_OK (0) or a negative bgtq_status.  No exception or abort
 *    crosses the ABI.  bgtq_last_error() returns a thread-local message for
 *    the last failure of the calling thread.
 *  - Arguments are validated on the host before anything is enqueued; a call
 *    that fails validation writes nothing.
 *  - Device pointers are caller-owned device allocations (the library never
 *    allocates device memory).  Host pointers are read during the call only.
 *  - Device work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream) with no host synchronisation, except where stated.
 *  - fp16 tensors are passed as uint16_t bit patterns (IEEE binary16).
 *  - head_dim is 128 (64 RoPE blocks) in this version.
 *  - A failed kernel launch returns BGTQ_EDEVICE.
 */
#ifndef BGTQ_H
#define BGTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bgtq_status;
enum {
  BGTQ_OK = 0,
  BGTQ_EINVAL = -1,     /* bad pointer, shape or flag */
  BGTQ_EBUDGET = -2,    /* bit budget outside 0..4 bits per coordinate */
  BGTQ_ECAPACITY = -3,  /* token range beyond the cache capacity */
  BGTQ_EDEVICE = -4,    /* HIP runtime or launch failure */
  BGTQ_EWORKSPACE = -5  /* workspace smaller than the size query */
};

#define BGTQ_ABI_VERSION 4
#define BGTQ_TILE 64 /* cache tokens per tile */

/* RoPE pairing of the 128 head coordinates into 64 2-D frequency blocks (the
 * pages name none; both conventions in use): half-split ("rotate-half"),
 * block j = coordinates (j, j+64); interleaved, block j = (2j, 2j+1). */
#define BGTQ_ROPE_HALF 0
#define BGTQ_ROPE_INTERLEAVED 1

typedef void *bgtq_stream; /* hipStream_t */

int32_t bgtq_abi_version(void);
const char *bgtq_last_error(void);

/*
 * (1) Label-free block energy (Abstract: "computes a label-free energy score
 * for each RoPE block"; README calibration paragraph: Q/K activations of one
 * forward pass).  Block j of a 128-wide head is the coordinate pair (a_j, b_j)
 * = (j, j+64) for rope_pairing BGTQ_ROPE_HALF, (2j, 2j+1) for
 * BGTQ_ROPE_INTERLEAVED.
 *   E[h][j] = Eq[h][j] * Ek[h][j]
 *   Eq[h][j] = sum over t < n_cal and h' in {hG..hG+G-1} of q[t][h'][a_j]^2 + q[t][h'][b_j]^2, / (n_cal G)
 *   Ek[h][j] = sum over t < n_cal of k[t][h][a_j]^2 + k[t][h][b_j]^2, / n_cal
 * Each sum is exact and rounded once to double; the division and the product
 * round once each, so the result is deterministic to the last bit.
 *   q_cal   device fp16 [n_cal][n_q_heads][head_dim], post-RoPE, d fastest
 *   k_cal   device fp16 [n_cal][n_kv_heads][head_dim]
 *   energy  device double [n_kv_heads][head_dim/2], written
 *   rope_pairing  BGTQ_ROPE_HALF or BGTQ_ROPE_INTERLEAVED
 * Eight workgroups per KV head (eight blocks each); the integer sums make the
 * result independent of how the tokens are split.
 * Errors: EINVAL on null pointers, q_cal or k_cal not 16-byte aligned, n_cal < 1
 * or n_cal > 2^22, head_dim != 128, n_q_heads not a positive multiple of
 * n_kv_heads (at most 1024 per KV head), an unknown rope_pairing.
 */
bgtq_status bgtq_energy(const uint16_t *q_cal, const uint16_t *k_cal, int64_t n_cal,
                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                        int32_t rope_pairing, double *energy, bgtq_stream stream);

/*
 * (2) Greedy integer bit allocation by marginal gain (Abstract: "greedily
 * allocates integer bit widths by marginal gain"; README introduction: bits
 * shift toward high-energy blocks under a fixed average budget).
 * Widths start at 0; avg_bits * n_blocks times, the block with the largest
 * gain E[j] * (D(b_j) - D(b_j + 1)) among blocks with b_j < 4 gets one more
 * bit (ties: lowest j).  D(b) is the b-bit Lloyd-Max MSE of N(0,1), D(0) = 1.
 * Host call, synchronous and deterministic: the greedy itself, run on the
 * caller's thread.
 *   energy  host double [n_kv_heads][n_blocks], finite and >= 0
 *   bits    host int8 [n_kv_heads][n_blocks], written (values 0..4)
 * Errors: EINVAL on null pointers, n_blocks != 64, n_kv_heads < 1 or an
 * energy that is negative or not finite; EBUDGET unless 0 <= avg_bits <= 4.
 * Nothing is written on an error.
 */
bgtq_status bgtq_allocate(const double *energy, int32_t n_kv_heads, int32_t n_blocks,
                          int32_t avg_bits, int8_t *bits);

/*
 * (2b) The same allocation on the device, for energies that are already in
 * device memory (the output of bgtq_energy): one wave per KV head takes the
 * avg_bits * 64 largest marginal gains in the order (gain descending, block
 * ascending, width ascending), which is the greedy's sequence of choices
 * because each block's gains do not increase with its width.  The result is
 * identical to bgtq_allocate's.
 *   energy  device double [n_kv_heads][n_blocks], finite and >= 0 (not checked)
 *   bits    device int8 [n_kv_heads][n_blocks], written
 * Errors: as bgtq_allocate except the energy check (the host cannot read it).
 */
bgtq_status bgtq_allocate_device(const double *energy, int32_t n_kv_heads, int32_t n_blocks,
                                 int32_t avg_bits, int8_t *bits, bgtq_stream stream);

/*
 * (3) Plan: everything the encoder and decoder need for one layer (Abstract:
 * Block-GTQ sits on top of TurboQuant-MSE, with integer widths per RoPE block
 * and KxVy budgets; README introduction: a per-(layer, KV head) allocation).
 * The pages fix neither TurboQuant-MSE's rotation nor its codebook; the plan
 * holds the readings taken.  Fixed by (widths, V width, seed, layer):
 * Lloyd-Max codebooks b = 1..4 in double, one seeded Haar rotation per
 * (KV head, K width group) and per KV head for V
 * (SplitMix64 stream absorbing seed, layer, kvh, tensor (K 0, V 1), width,
 * group size; Box-Muller; Householder QR with the sign of diag(R) taken
 * positive), the group maps, the bit offsets of the key stream and the
 * decode tables.  Plans are immutable; one plan may be used
 * from several threads and streams at once.
 */
typedef struct bgtq_plan bgtq_plan;

typedef struct {
  int32_t n_kv_heads;
  int32_t n_q_heads;    /* G = n_q_heads / n_kv_heads query heads per KV head, 1 <= G <= 8;
                           query head h reads KV head h / G */
  int32_t head_dim;     /* 128 */
  int32_t k_avg_bits;   /* 0..4; each row of k_bits must sum to k_avg_bits * 64 */
  int32_t v_bits;       /* 1..4 */
  const int8_t *k_bits; /* host int8 [n_kv_heads][64], values 0..4 */
  uint64_t seed;
  int32_t layer;
  int32_t rope_pairing; /* BGTQ_ROPE_HALF (0) or BGTQ_ROPE_INTERLEAVED: the two coordinates that block j
                           contributes to its key group */
} bgtq_plan_desc;

typedef struct {
  uint64_t consts;  /* device constant image written by bgtq_plan_upload */
  uint64_t k_codes; /* u32 [batch][Hkv][tiles][4*k_avg_bits][64] */
  uint64_t k_norms; /* fp16 [batch][Hkv][tiles][64][4], slot 4-w holds the width-w group norm */
  uint64_t v_codes; /* u32 [batch][Hkv][tiles][128][2*v_bits] */
  uint64_t v_norms; /* fp16 [batch][Hkv][tiles][64] */
} bgtq_sizes;

/* Errors: EINVAL (null, shape, unknown rope_pairing), EBUDGET (a row of k_bits does not sum to
 * k_avg_bits * 64 or holds a width outside 0..4, v_bits outside 1..4). */
bgtq_status bgtq_plan_create(const bgtq_plan_desc *desc, bgtq_plan **out);
void bgtq_plan_destroy(bgtq_plan *plan);

/* Byte sizes of the constant image and of the cache arrays for `batch`
 * sequences of `capacity` tokens (tiles = ceil(capacity / 64)). The caller
 * zero-fills the cache arrays before the first encode. */
bgtq_status bgtq_plan_sizes(const bgtq_plan *plan, int32_t batch, int64_t capacity,
                            bgtq_sizes *out);

/* Copies the constant image into caller memory `dev_consts` (sizes.consts
 * bytes, 256-byte aligned) on `stream`.  The plan must outlive the copy. */
bgtq_status bgtq_plan_upload(const bgtq_plan *plan, void *dev_consts, bgtq_stream stream);

/*
 * (4) TurboQuant-MSE encode of n_new tokens at positions t0 .. t0+n_new-1 of
 * every sequence (prefill: t0 = 0; append: t0 = current length).  Abstract:
 * keys are quantised block group by block group at the allocated widths on a
 * TurboQuant-MSE encoder, values at a uniform width (the "V" of KxVy); the
 * pages leave the encoder's steps open, and the ones below are the readings
 * taken.  Per token,
 * KV head and width group: n = ||x_g|| (exact sum of squares, rounded once,
 * correctly rounded sqrt), y = Pi x_g / n (0 if n = 0), z = sqrt(d_g) y,
 * code_i = #{Lloyd-Max thresholds < z_i}; the norm is stored as fp16 with one
 * round-to-nearest-even step.  Keys use the plan's widths (groups in width
 * order 4,3,2,1, each block's two coordinates adjacent (j, j+64 or 2j, 2j+1
 * by the plan's rope_pairing), blocks ascending); values one group of all 128
 * coordinates at v_bits.
 *   k / v      device fp16 [batch][n_new][n_kv_heads][128], post-RoPE keys,
 *              16-byte aligned
 *   capacity   tokens per sequence the cache arrays were sized for
 *   k_codes... device arrays laid out as in bgtq_sizes
 * Tokens outside [t0, t0+n_new) are left unchanged.
 * Errors: EINVAL (null, batch < 1, n_new < 0, k / v not 16-byte aligned),
 * ECAPACITY (t0 < 0 or t0 + n_new > capacity).
 */
bgtq_status bgtq_encode_k(const bgtq_plan *plan, const void *dev_consts, const uint16_t *k,
                          int32_t batch, int64_t capacity, int64_t t0, int64_t n_new,
                          uint32_t *k_codes, uint16_t *k_norms, bgtq_stream stream);
bgtq_status bgtq_encode_v(const bgtq_plan *plan, const void *dev_consts, const uint16_t *v,
                          int32_t batch, int64_t capacity, int64_t t0, int64_t n_new,
                          uint32_t *v_codes, uint16_t *v_norms, bgtq_stream stream);

/* (4) for keys and values of the same tokens in one call: the caches are
 * written exactly as bgtq_encode_k followed by bgtq_encode_v would write them
 * (same codes and norms, bit for bit).  Where the tiles of the range times
 * KV heads times sequences are at most the compute-unit count (an append of a
 * few thousand tokens), the two encodes run in one launch, side by side;
 * larger encodes run them one after the other.
 * Arguments, errors and the 16-byte alignment of k and v as bgtq_encode_k/v.
 */
bgtq_status bgtq_encode_kv(const bgtq_plan *plan, const void *dev_consts, const uint16_t *k, const uint16_t *v,
                           int32_t batch, int64_t capacity, int64_t t0, int64_t n_new, uint32_t *k_codes,
                           uint16_t *k_norms, uint32_t *v_codes, uint16_t *v_norms, bgtq_stream stream);

/*
 * (5) Query rotation (the fused decode's query side; Abstract: logits are
 * sums over RoPE frequency blocks, and a TurboQuant-MSE code lives in its
 * group's rotated space, so q is rotated once per key group instead of
 * un-rotating every key): for every query head h and present key width group g,
 * q_rot[b][h][o_g + i] = sum_k Pi_g[i][k] q[b][h][coord_g[k]] (fp32, matrix
 * cores), o_g = sum of the sizes of the groups before g; entries past the
 * last group are 0.  This is the "rotate q once per group" step of the fused
 * decode (logits are taken in the rotated space).
 *   q      device fp16 [batch][n_q_heads][128] (post-RoPE)
 *   q_rot  device float [batch][n_q_heads][128], written
 */
bgtq_status bgtq_rotate_queries(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                int32_t batch, float *q_rot, bgtq_stream stream);

/*
 * (5k) Key logits from the packed key cache alone (K-only).  Abstract: the
 * method is judged by the error of the RoPE query-key logits with only the
 * keys quantised (2 and 3 bits per coordinate); the README's per-layer
 * diagnostic takes it over the last positions of a layer.  For every
 * sequence b, query n < n_q, query head h and token t < n_k,
 *   logits[b][h][n][t] = q[b][n][h] . k_hat[b][t0 + t][h / G]   (unscaled)
 * with k_hat the TurboQuant-MSE reconstruction of the cached key, taken in the
 * rotated space of each key group: sum_g n_g sum_i q_rot_g,i c_w[code_i] /
 * sqrt(d_g), fp32.
 *   q_rot   device float [batch][n_q][n_q_heads][128]: bgtq_rotate_queries of
 *           the fp16 queries [batch][n_q][n_q_heads][128] called with batch x
 *           n_q sequences
 *   k_codes, k_norms  the key arrays of a contiguous cache of `capacity`
 *           tokens (bgtq_sizes); k_codes may be null for a plan without key bits
 *   logits  device float [batch][n_q_heads][n_q][n_k], written
 * Errors: EINVAL (null, batch outside 1..65535, n_q < 1), ECAPACITY (t0 < 0,
 * n_k < 0 or t0 + n_k > capacity).  n_k = 0 writes nothing.
 */
bgtq_status bgtq_key_logits(const bgtq_plan *plan, const void *dev_consts, const float *q_rot, int32_t n_q,
                            const uint32_t *k_codes, const uint16_t *k_norms, int64_t capacity,
                            int32_t batch, int64_t t0, int64_t n_k, float *logits, bgtq_stream stream);

/*
 * (6) Fused decode attention over the packed cache for one new query per
 * sequence (the packed-cache serving path of the Abstract and the README
 * backend table): per (sequence, query head),
 *   l_t = softmax_scale * q . k_hat_t,  o = sum_t softmax(l)_t v_hat_t
 * over t < seq_len, where k_hat, v_hat are the TurboQuant-MSE reconstructions
 * (fp16 norm * Pi^T (centroid / sqrt(d_g))).  Computed without
 * materialising k_hat or v_hat, in three launches: a preparation kernel
 * rotates the queries once per key group; the decode kernel takes the logits
 * in the rotated space from LDS centroid lookups on the matrix cores (fp32
 * products for the 4-bit group -- with eight query heads per KV head, query and
 * centroid each split into two fp16 parts -- and fp16 operands for widths
 * 1..3), keeps an online softmax and accumulates the values in the rotated
 * value space, one partial per split of the sequence; the merge kernel
 * combines the splits and un-rotates once per head.  fp32 accumulation
 * throughout.  The value operand (softmax
 * weight x fp16 value norm) is kept finite for every finite value norm (the
 * running maximum is raised early for tokens whose norm is 128 or more); a
 * value whose norm overflowed fp16 at encode (+inf) makes the output NaN, as
 * its reconstruction is infinite.
 *   q           device fp16 [batch][n_q_heads][128]
 *   seq_lens    device int32 [batch]; each value is clamped to [0, max_seq_len];
 *               a sequence of length 0 yields a zero output
 *   max_seq_len host bound on every seq_lens entry, 1 <= max_seq_len <= capacity
 *   out         device fp16 [batch][n_q_heads][128], written
 *   workspace   device scratch of at least bgtq_decode_workspace_size bytes
 * Errors: EINVAL, ECAPACITY (max_seq_len outside [1, capacity]),
 * EWORKSPACE (ws_bytes too small).
 */
bgtq_status bgtq_decode_workspace_size(const bgtq_plan *plan, int32_t batch, int64_t max_seq_len,
                                       size_t *bytes);
bgtq_status bgtq_decode_attn(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                             const uint32_t *k_codes, const uint16_t *k_norms,
                             const uint32_t *v_codes, const uint16_t *v_norms, int64_t capacity,
                             const int32_t *seq_lens, int32_t batch, int64_t max_seq_len,
                             float softmax_scale, uint16_t *out, void *workspace, size_t ws_bytes,
                             bgtq_stream stream);

/*
 * (6n) bgtq_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials go to a scratch array
 * the library holds in device memory (bgtq_noalloc_scratch_bytes() bytes,
 * 4 MiB, one per device, kept until the process ends); the call makes no HIP
 * allocation of any kind.  Every call on a device shares that device's
 * scratch, which needs no clearing (each call writes the partials it reads):
 * calls that overlap on one device (other streams, other threads) race and
 * must not be issued.  Results are identical to bgtq_decode_attn's.
 * Arguments as bgtq_decode_attn without workspace and ws_bytes.
 * Errors: as bgtq_decode_attn; EWORKSPACE when the partials
 * (bgtq_decode_workspace_size) exceed the scratch.
 */
size_t bgtq_noalloc_scratch_bytes(void);
bgtq_status bgtq_decode_attn_noalloc(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                     const uint32_t *k_codes, const uint16_t *k_norms,
                                     const uint32_t *v_codes, const uint16_t *v_norms, int64_t capacity,
                                     const int32_t *seq_lens, int32_t batch, int64_t max_seq_len,
                                     float softmax_scale, uint16_t *out, bgtq_stream stream);

/*
 * (6b) Decode attention with an fp16 sink and recent window: the Block-GTQ
 * README runs its AIME evaluation in two settings, without and with an fp16
 * buffer of 4 attention-sink tokens and a 128-token recent window.  Reading
 * taken: for a sequence of length T, token t attends with its original fp16
 * key and value when t < n_sink or t >= T - n_recent, and through the packed
 * cache otherwise; the softmax runs over all T tokens.  The packed cache
 * still holds every token (so a token leaving the window needs no
 * re-encoding); the decode kernel skips the buffered ones and the merge
 * kernel takes the fp16 tokens itself, in parallel with the split partials.
 *   k_sink, v_sink      device fp16 [batch][n_kv_heads][n_sink][128], token t < n_sink in row t
 *   k_recent, v_recent  device fp16 [batch][n_kv_heads][n_recent][128], token t in row t % n_recent
 *                       (a ring: it must hold tokens [max(0, T - n_recent), T))
 *   n_sink              0..64;  n_recent 0..65536
 *   everything else     as bgtq_decode_attn (the same workspace size)
 * Null buffer pointers are allowed for a zero count.  n_sink = n_recent = 0 is
 * bgtq_decode_attn.
 * Errors: as bgtq_decode_attn; EINVAL for counts out of range or a null
 * buffer with a non-zero count.
 */
bgtq_status bgtq_decode_attn_buffered(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                      const uint32_t *k_codes, const uint16_t *k_norms,
                                      const uint32_t *v_codes, const uint16_t *v_norms, int64_t capacity,
                                      const int32_t *seq_lens, int32_t batch, int64_t max_seq_len,
                                      float softmax_scale, const uint16_t *k_sink, const uint16_t *v_sink,
                                      int32_t n_sink, const uint16_t *k_recent, const uint16_t *v_recent,
                                      int32_t n_recent, uint16_t *out, void *workspace, size_t ws_bytes,
                                      bgtq_stream stream);

/*
 * (6c) Buffer append: copies new fp16 keys and values into the sink and
 * recent-window buffers of (6b).  Token t = t0 + i (i < n_new) goes to sink
 * row t when t < n_sink and to ring row t % n_recent when
 * t >= t0 + n_new - n_recent (earlier new tokens would be overwritten by later
 * ones of the same call).  Call it with the same k/v as bgtq_encode_k/v.
 *   k, v     device fp16 [batch][n_new][n_kv_heads][128]
 *   buffers  as (6b), written
 * Errors: EINVAL on null pointers with non-zero counts, counts out of range,
 * t0 < 0 or n_new < 0.
 */
bgtq_status bgtq_buffer_append(const uint16_t *k, const uint16_t *v, int32_t batch, int64_t n_new, int64_t t0,
                               int32_t n_kv_heads, uint16_t *k_sink, uint16_t *v_sink, int32_t n_sink,
                               uint16_t *k_recent, uint16_t *v_recent, int32_t n_recent, bgtq_stream stream);

/*
 * (6d) Paged packed cache (the paged-KV serving layout: the cache as a pool of
 * fixed-size pages and a per-sequence block table, so that sequences grow
 * without reallocation and share one pool).  The pages name a packed-cache
 * serving path (Abstract; README backend table) but no cache organisation;
 * the paged form is the one serving engines use.  A page is one 64-token tile of
 * one KV head; the pool arrays are the per-tile blocks of (4) with the pages
 * in place of the tiles:
 *   k_codes  u32  [n_kv_heads][n_pages][4*k_avg_bits][64]
 *   k_norms  fp16 [n_kv_heads][n_pages][64][4]
 *   v_codes  u32  [n_kv_heads][n_pages][128][2*v_bits]
 *   v_norms  fp16 [n_kv_heads][n_pages][64]
 * (bgtq_plan_sizes(plan, 1, 64 * n_pages) gives their sizes).  Token t of
 * sequence b lives in page block_table[b][t / 64], row t % 64, for every KV
 * head.  The table is read on the device; entries must lie in [0, n_pages)
 * for every tile a call writes or attends to (an entry outside the pool makes
 * the writers skip that tile; reads are clamped to the pool, so a bad entry
 * gives wrong results, never an access outside the pool).  Decoding a paged
 * pool gives the same results, bit for bit, as the contiguous cache holding
 * the same tokens.
 */
typedef struct {
  const int32_t *block_table; /* device int32 [batch][max_pages] */
  int32_t max_pages;          /* table entries per sequence: capacity 64 * max_pages tokens */
  int32_t n_pages;            /* pages in the pool */
} bgtq_pages;

/* (4) on a paged pool: tokens t0 .. t0 + n_new - 1 of every sequence, k / v as
 * in (4).  Errors: as (4), with capacity = 64 * max_pages; EINVAL for null
 * pages or table, max_pages < 1 or n_pages < 1. */
bgtq_status bgtq_encode_k_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *k,
                                int32_t batch, const bgtq_pages *pages, int64_t t0, int64_t n_new,
                                uint32_t *k_codes, uint16_t *k_norms, bgtq_stream stream);
bgtq_status bgtq_encode_v_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *v,
                                int32_t batch, const bgtq_pages *pages, int64_t t0, int64_t n_new,
                                uint32_t *v_codes, uint16_t *v_norms, bgtq_stream stream);
/* bgtq_encode_kv on a paged pool: as bgtq_encode_k_paged followed by
 * bgtq_encode_v_paged. */
bgtq_status bgtq_encode_kv_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *k,
                                 const uint16_t *v, int32_t batch, const bgtq_pages *pages, int64_t t0,
                                 int64_t n_new, uint32_t *k_codes, uint16_t *k_norms, uint32_t *v_codes,
                                 uint16_t *v_norms, bgtq_stream stream);

/* (6) on a paged pool: everything as bgtq_decode_attn, capacity 64 * max_pages
 * (the same workspace size).  Errors: as (6); EINVAL for bad pages. */
bgtq_status bgtq_decode_attn_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                   const uint32_t *k_codes, const uint16_t *k_norms,
                                   const uint32_t *v_codes, const uint16_t *v_norms,
                                   const bgtq_pages *pages, const int32_t *seq_lens, int32_t batch,
                                   int64_t max_seq_len, float softmax_scale, uint16_t *out,
                                   void *workspace, size_t ws_bytes, bgtq_stream stream);

/* (6) on a paged pool with the fp16 sink and recent window (6b): the packed
 * tokens are read through the block table as in bgtq_decode_attn_paged, the
 * buffered ones from the fp16 buffers as in bgtq_decode_attn_buffered.
 * Arguments and errors: those two calls'. */
bgtq_status bgtq_decode_attn_paged_buffered(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                            const uint32_t *k_codes, const uint16_t *k_norms,
                                            const uint32_t *v_codes, const uint16_t *v_norms,
                                            const bgtq_pages *pages, const int32_t *seq_lens, int32_t batch,
                                            int64_t max_seq_len, float softmax_scale, const uint16_t *k_sink,
                                            const uint16_t *v_sink, int32_t n_sink, const uint16_t *k_recent,
                                            const uint16_t *v_recent, int32_t n_recent, uint16_t *out,
                                            void *workspace, size_t ws_bytes, bgtq_stream stream);

/*
 * (7) Decode step: appends one new key and value per sequence to the packed
 * cache and attends the new query over the cache including that token (the
 * serving step of the packed-cache path, Abstract and README backend table:
 * each generated token is encoded into the packed cache and the fused kernel
 * attends over it).  For
 * each sequence b with 0 <= pos[b] < capacity, k_new[b] and v_new[b] are
 * encoded at token pos[b] exactly as bgtq_encode_k / bgtq_encode_v would
 * (sequences with pos[b] outside that range append nothing); then the output
 * is bgtq_decode_attn's with seq_lens[b] = pos[b] + 1 (clamped to
 * [0, max_seq_len]).  One append launch, then the two decode launches.
 *   q            device fp16 [batch][n_q_heads][128]
 *   k_new, v_new device fp16 [batch][n_kv_heads][128]
 *   pos          device int32 [batch]
 *   caches       as for bgtq_encode_k / bgtq_encode_v (written) and bgtq_decode_attn (read)
 *   workspace    bgtq_decode_workspace_size(plan, batch, max_seq_len) bytes, 256-byte aligned
 * Errors: as bgtq_decode_attn.
 */
bgtq_status bgtq_decode_step(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                             const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos, int32_t batch,
                             int64_t max_seq_len, uint32_t *k_codes, uint16_t *k_norms, uint32_t *v_codes,
                             uint16_t *v_norms, int64_t capacity, float softmax_scale, uint16_t *out,
                             void *workspace, size_t ws_bytes, bgtq_stream stream);

/* (7) with the fp16 sink and recent window (6b): the new token of sequence b is
 * appended to the packed cache as in bgtq_decode_step and copied into the
 * buffers as bgtq_buffer_append would copy token pos[b] (sink row pos[b] when
 * below n_sink, ring row pos[b] % n_recent; nothing for pos[b] < 0), then the
 * output is bgtq_decode_attn_buffered's over pos[b] + 1 tokens.
 *   k_sink ... n_recent   as for bgtq_decode_attn_buffered (written, then read)
 * Errors: as bgtq_decode_step and bgtq_decode_attn_buffered. */
bgtq_status bgtq_decode_step_buffered(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                      const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                      int32_t batch, int64_t max_seq_len, uint32_t *k_codes, uint16_t *k_norms,
                                      uint32_t *v_codes, uint16_t *v_norms, int64_t capacity, float softmax_scale,
                                      uint16_t *k_sink, uint16_t *v_sink, int32_t n_sink, uint16_t *k_recent,
                                      uint16_t *v_recent, int32_t n_recent, uint16_t *out, void *workspace,
                                      size_t ws_bytes, bgtq_stream stream);

/* (7) on a paged pool (6d): the new token of sequence b goes to page
 * block_table[b][pos[b] / 64] (sequences with pos[b] outside
 * [0, 64 * max_pages) append nothing), then bgtq_decode_attn_paged over
 * pos[b] + 1 tokens.  Errors: as bgtq_decode_attn_paged. */
bgtq_status bgtq_decode_step_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                   const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                   int32_t batch, int64_t max_seq_len, uint32_t *k_codes, uint16_t *k_norms,
                                   uint32_t *v_codes, uint16_t *v_norms, const bgtq_pages *pages,
                                   float softmax_scale, uint16_t *out, void *workspace, size_t ws_bytes,
                                   bgtq_stream stream);

/*
 * (8) fp16 decode attention over an uncompressed KV cache: the baseline of the
 * packed path (Abstract: the packed path runs faster than fp16
 * FlashAttention-2 decode at 128K; README end-to-end decode benchmark).  Per
 * (sequence, query head h, KV head h / G):
 *   o = sum_{t < seq_len} softmax(softmax_scale * q . k_t)_t v_t
 * with fp16 inputs, fp32 products and sums, fp16 output; two launches (split
 * stream, split merge), the same structure as bgtq_decode_attn.
 *   q         device fp16 [batch][n_q_heads][128], 16-byte aligned
 *   k, v      device fp16 [batch][capacity][n_kv_heads][128], 16-byte aligned
 *   seq_lens  device int32 [batch], clamped to [0, max_seq_len]; length 0 gives 0
 *   out       device fp16 [batch][n_q_heads][128], written
 *   workspace bgtq_fp16_decode_workspace_size bytes, 256-byte aligned
 * Errors: EINVAL (null, shapes, G not 1, 2, 4 or 8, alignment, scale),
 * ECAPACITY (max_seq_len outside [1, capacity]), EWORKSPACE.
 */
bgtq_status bgtq_fp16_decode_workspace_size(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                            int64_t max_seq_len, size_t *bytes);
bgtq_status bgtq_fp16_decode_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v, int32_t batch,
                                  int32_t n_q_heads, int32_t n_kv_heads, int64_t capacity,
                                  const int32_t *seq_lens, int64_t max_seq_len, float softmax_scale,
                                  uint16_t *out, void *workspace, size_t ws_bytes, bgtq_stream stream);

/*
 * Host-side inspection (no device work).
 * bgtq_codebook: the b-bit Lloyd-Max quantiser of N(0,1) the library uses:
 * centroids [2^b], interior thresholds [2^b - 1], and D(b).
 * bgtq_plan_rotation: the plan's rotation for (kvh, tensor 0 = K / 1 = V,
 * width) into out [d*d] row-major (Pi[i][k]); *dim receives d (0 if the width
 * is absent).  out may be NULL to query d only.
 * bgtq_plan_bits: the plan's widths [n_kv_heads][64].
 */
bgtq_status bgtq_codebook(int32_t bits, double *centroids, double *thresholds, double *distortion);
bgtq_status bgtq_plan_rotation(const bgtq_plan *plan, int32_t kvh, int32_t tensor, int32_t width,
                               double *out, int32_t *dim);
bgtq_status bgtq_plan_bits(const bgtq_plan *plan, int8_t *bits);

/*
 * Kernel timing: when enabled, bgtq_decode_attn and bgtq_decode_step bind HIP
 * events to every launch of their decode kernel on `stream`; bgtq_profile_read waits for the
 * recorded events, returns the summed duration (ms) and launch count since
 * the last read, and clears them.
 */
bgtq_status bgtq_profile_enable(int32_t on);
bgtq_status bgtq_profile_read(double *stream_kernel_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* BGTQ_H */
