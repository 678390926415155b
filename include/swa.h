/*
 * swa.h - C ABI of the gfx950 (MI355X) sliding-window attention library.
 *
 * Sliding-window attention (SWA): query i attends only to the keys inside a
 * fixed window around it, with the softmax taken over the in-window logits
 * (every out-of-window logit counts as -inf).  Sources:
 *   - robocikowo.com glossary "Sliding Window Attention", opening definition:
 *     causal window [i-W+1, i], symmetric window [i-W/2, i+W/2], masked logits
 *     set to -inf before the softmax;
 *   - Ultralytics glossary "Sliding Window Attention", section "Come cresce la
 *     finestra con la profondita": the causal mask 0 <= i-j < w, and the
 *     w-slot circular KV buffer that stores position i in slot i mod w;
 *   - aivaro.ru answer 629, section 4.1: the Longformer window takes W/2
 *     neighbours on each side;
 *   - "Sliding-window and hybrid attention", section "Walking through it":
 *     windowed decode reads only the window's KV for each new token;
 *   - aivaro.ru answer 629, sections 4.2 and 4.3: the dilated window and the
 *     global tokens of Longformer;
 *   - Ultralytics glossary, terms section: attention sinks kept beside the
 *     window (StreamingLLM).
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, contiguous and head-major:
 *       q, out        [B, Hq,  T, d]   (prefill)      [B, Hq, d]   (decode)
 *       k, v          [B, Hkv, T, d]
 *       k_ring, v_ring[B, Hkv, W, d]
 *       k_new, v_new  [B, Hkv, d]
 *       pos           [B] int32
 *     and for a chunk of n tokens per sequence (chunked prefill)
 *       q, out        [B, Hq, n, d]    k, v  [B, Hkv, n, d]
 *     attention sinks beside a ring: k_sink, v_sink [B, Hkv, S, d];
 *     global token positions: global_pos [G] int32.
 *     Element type is selected by `dtype` (swa_dtype): IEEE fp32 or bfloat16.
 *   - Query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups); Hq
 *     must be a multiple of Hkv.
 *   - Every pointer is a device pointer the caller owns.  The library never
 *     allocates or frees memory and keeps no state between calls.  Every
 *     device pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; calls are thread-safe.
 *   - Arguments are validated on the host before anything is enqueued.  An
 *     invalid call returns a negative swa_status and launches nothing; a
 *     failed launch returns SWA_ERR_LAUNCH (for the calls made of two or
 *     three kernels, the ones before the failure may already be enqueued, and
 *     the output is then undefined).  Device-side contents (e.g. pos)
 *     are not validated on the host; the behaviour for out-of-range positions
 *     is stated per entry point and never touches memory outside the buffers.
 *   - Accumulation and softmax run in fp32; bf16 outputs are rounded to
 *     nearest-even.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SWA_OK = 0,
  SWA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, Hq % Hkv != 0,
                               scale not finite or |scale| > 1024, misaligned
                               pointer */
  SWA_ERR_UNSUPPORTED = -2, /* d not in {32, 64, 128}, unknown mode or dtype,
                               sequence longer than 2^29, launch grid beyond
                               the int32 range */
  SWA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  SWA_ERR_LAUNCH = -4       /* the HIP runtime rejected a kernel launch */
} swa_status;

typedef enum {
  SWA_CAUSAL = 0,   /* keys j with 0 <= i - j <= W - 1                        */
  SWA_SYMMETRIC = 1 /* keys j with |i - j| <= floor(W / 2); W + 1 keys inside
                       the sequence when W is even                           */
} swa_mode;

typedef enum { SWA_F32 = 0, SWA_BF16 = 1 } swa_dtype;

/*
 * swa_prefill - windowed attention over a whole sequence (every query row).
 *
 *   out[b,h,i,:] = sum_j softmax_j(scale * q[b,h,i,:].k[b,g,j,:]) v[b,g,j,:]
 *   over the keys j in the window of i (mode), clipped to 0 <= j < T,
 *   g = h / (Hq / Hkv).
 *
 * Causal window from the robocikowo definition and the Ultralytics mask
 * snippet; symmetric window from the robocikowo definition and aivaro
 * section 4.1.  Only key tiles that intersect the window are visited; the
 * [T, T] score matrix is never formed.
 *
 * Batch is folded into the heads: for tensors [B, H, T, d] pass Hq = B*Hq_model
 * and Hkv = B*Hkv_model (exact, because B*Hq_model/(B*Hkv_model) keeps the
 * group size and b*Hq_model + h maps to b*Hkv_model + h/group).
 *
 *   q, k, v  input, layouts above, element type `dtype`.
 *   out      output [Hq, T, d] (may not alias q, k or v).
 *   T >= 1, W >= 1, Hq >= 1, Hkv >= 1, Hq % Hkv == 0, d in {32, 64, 128},
 *   mode in swa_mode, |scale| <= 1024 (SWA_ERR_INVALID_ARG otherwise; see
 *   below), dtype in swa_dtype; T <= 2^29 (SWA_ERR_UNSUPPORTED otherwise).
 *   W may exceed T: W >= T (causal) or floor(W/2) >= T - 1 (symmetric) is full
 *   attention.
 * Scale bound (every entry point): the softmax exponent scale*log2(e)*(s - m)
 * is formed in fp32 as s*c - m*c, whose rounding grows with |s * c|; up to
 * |scale| = 1024 it stays below 0.01 for scores up to 100 in magnitude.
 * Returns SWA_OK or a negative swa_status.
 */
int swa_prefill(const void* q, const void* k, const void* v, void* out, int T, int W, int Hq,
                int Hkv, int d, int mode, float scale, int dtype, void* stream);

/*
 * swa_prefill_dilated - windowed attention with a dilated window.
 *
 * Key j is in the window of query i when i - j is a multiple of `dilation`
 * and m = (i - j) / dilation lies in the plain window of `mode` (causal
 * 0 <= m <= W-1; symmetric |m| <= floor(W/2)), clipped to 0 <= j < T.  The
 * window keeps its number of keys and spreads them `dilation` apart
 * (aivaro.ru answer 629, section 4.2: W = 512 at dilation 2 gives 256 keys
 * each side over 1024 positions; robocikowo glossary, dilated-SWA variant:
 * gaps as in a dilated convolution).  dilation = 1 is swa_prefill.
 *
 *   Arguments, layouts and errors as swa_prefill, plus
 *   dilation >= 1 (SWA_ERR_INVALID_ARG otherwise); dilation * d * element
 *   size * 64 < 2^31 (SWA_ERR_UNSUPPORTED otherwise).
 */
int swa_prefill_dilated(const void* q, const void* k, const void* v, void* out, int T, int W,
                        int Hq, int Hkv, int d, int mode, float scale, int dilation, int dtype,
                        void* stream);

/*
 * swa_prefill_global - windowed attention plus global tokens.
 *
 * aivaro.ru answer 629, section 4.3 (Longformer global attention) and the
 * robocikowo glossary's global-tokens entry: a few chosen tokens attend to
 * every token, and every token attends to them, on top of the sliding
 * window.  With G global positions p_1 < ... < p_G:
 *   - a global row i = p_t attends to every key j (j <= i when causal);
 *   - any other row i attends to its window plus the global keys
 *     (those with j <= i when causal).
 * Causal global tokens at the first positions are attention sinks.
 * G = 0 is swa_prefill.  The same positions apply to every sequence of the
 * batch (batch folded into the heads as for swa_prefill).
 *
 * Computed in passes on `stream`: the windowed kernel visits the global
 * keys as extra tiles (skipping those inside a row's window), then a split-K
 * pass over the whole sequence writes partials of the G global rows (bf16: on
 * the matrix cores, 128 keys per split; fp32: the split-K kernel of
 * swa_decode), merged into those rows of `out`.
 *
 *   Arguments, layouts and errors as swa_prefill, plus
 *   global_pos  device int32 [G], strictly increasing positions in [0, T)
 *               (not checked on the host; entries outside [0, T) are
 *               ignored, repeated or unsorted entries give unspecified rows,
 *               never an access outside the buffers).  May be NULL when G = 0.
 *   G >= 0.
 *   workspace   device scratch of at least
 *               swa_prefill_global_workspace_bytes(T, Hq, G, d) bytes when
 *               G > 0 (partials of the global rows); no initialisation
 *               needed; concurrent calls need distinct workspaces.
 *               SWA_ERR_WORKSPACE if missing or too small.
 *   T * d * element size < 2^31.
 */
int swa_prefill_global(const void* q, const void* k, const void* v, void* out, int T, int W,
                       int Hq, int Hkv, int d, int mode, float scale, const int32_t* global_pos,
                       int G, void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * swa_prefill_dilated_global - dilated window plus global tokens.
 *
 * aivaro.ru answer 629, sections 4.2 and 4.3: Longformer combines the two.
 * A non-global row i attends to its dilated window (keys i - m * dilation
 * for m in the plain window's offsets, as swa_prefill_dilated) plus the
 * global keys not already in it (j <= i when causal); a global row attends
 * to every key (j <= i when causal), as in swa_prefill_global.
 * dilation = 1 is swa_prefill_global; G = 0 is swa_prefill_dilated.
 *
 *   Arguments, layouts, workspace and errors as swa_prefill_global, plus
 *   dilation >= 1 (SWA_ERR_INVALID_ARG otherwise), with
 *   64 * dilation * d * element size < 2^31 (SWA_ERR_UNSUPPORTED).
 */
int swa_prefill_dilated_global(const void* q, const void* k, const void* v, void* out, int T,
                               int W, int Hq, int Hkv, int d, int mode, float scale, int dilation,
                               const int32_t* global_pos, int G, void* workspace,
                               size_t workspace_bytes, int dtype, void* stream);

/*
 * swa_cache_append - write one new K/V row per sequence into the ring cache.
 *
 *   k_ring[b, :, pos[b] mod W, :] = k_new[b, :, :]   (and the same for v)
 *
 * Ultralytics ring-buffer paragraph (slot i mod w, the oldest entry is
 * overwritten); robocikowo rolling KV buffer (FIFO over the last W tokens).
 * A bit-exact copy.  A sequence with pos[b] < 0 is left untouched.
 *
 *   k_ring, v_ring  in/out [B, Hkv, W, d].
 *   pos             device int32 [B], the position of the new token.
 *   k_new, v_new    input [B, Hkv, d].
 *   B, Hkv, W >= 1, d in {32, 64, 128}, dtype in swa_dtype.
 */
int swa_cache_append(void* k_ring, void* v_ring, const int32_t* pos, const void* k_new,
                     const void* v_new, int B, int Hkv, int W, int d, int dtype, void* stream);

/*
 * swa_decode - one query token per sequence against its ring cache (causal).
 *
 * The query at position p = pos[b] sees positions [max(0, p-W+1), p], held in
 * slots p' mod W, i.e. the slots [0, min(p+1, W)).  Call swa_cache_append for
 * position p first, so that the query sees its own key.  Equals row p of
 * swa_prefill (causal, same W) over the sequence that filled the ring.
 * "Sliding-window and hybrid attention", section "Walking through it": each
 * decoded token reads at most W cached rows rather than the whole history.
 * A sequence with pos[b] < 0 gets an all-zero output row.
 *
 *   q          input [B, Hq, d].
 *   k_ring, v_ring  input [B, Hkv, W, d].
 *   pos        device int32 [B].
 *   out        output [B, Hq, d].
 *   workspace  device scratch of at least swa_decode_workspace_bytes(B, Hq, W, d)
 *              bytes (partial results of the split-K passes); its contents
 *              need no initialisation and are garbage afterwards.  Concurrent
 *              calls must use distinct workspaces.
 *   mode is implicitly causal: there is no symmetric decode (the symmetric
 *   window needs keys that have not been generated yet).
 */
int swa_decode(const void* q, const void* k_ring, const void* v_ring, const int32_t* pos,
               void* out, int B, int Hq, int Hkv, int W, int d, float scale, int dtype,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * swa_decode_noalloc - swa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * Same computation, arguments, layouts and errors as swa_decode, without the
 * workspace: when the ring is split, the split partials go to a scratch
 * array the library holds on each GPU (one copy per device, kept until the
 * process ends, at most 4 MiB; every call on that device shares it).  The
 * call allocates nothing and needs no initialisation; partials are written
 * before the same call reads them.  Calls that overlap in time on one GPU
 * (other streams, other threads) race on the scratch and give undefined
 * outputs: serialise them.  A call whose partials would not fit returns
 * SWA_ERR_UNSUPPORTED (no valid size does today: at most 4096 records of
 * d + 2 floats); failing to find the scratch's device address returns
 * SWA_ERR_LAUNCH.
 */
int swa_decode_noalloc(const void* q, const void* k_ring, const void* v_ring, const int32_t* pos,
                       void* out, int B, int Hq, int Hkv, int W, int d, float scale, int dtype,
                       void* stream);

/*
 * swa_cache_append_chunk - append n consecutive tokens per sequence to the
 * ring cache.
 *
 *   token i of sequence b has position pos[b] + i and is written to slot
 *   (pos[b] + i) mod W:  k_ring[b, :, (pos[b]+i) mod W, :] = k[b, :, i, :]
 *   (and the same for v).
 *
 * The result equals n single appends in order (Ultralytics ring-buffer
 * paragraph: slot i mod w, the oldest entry is overwritten), so when n > W
 * only the last W tokens of the chunk remain; the earlier ones are not
 * written at all.  A bit-exact copy.  A sequence with pos[b] < 0 is left
 * untouched.  Positions pos[b] + n - 1 must stay below 2^31; a larger value
 * lands in some slot of its own sequence, never outside the ring.
 *
 *   k_ring, v_ring  in/out [B, Hkv, W, d].
 *   pos             device int32 [B], the position of each chunk's first token.
 *   k, v            input [B, Hkv, n, d].
 *   B, n, Hkv, W >= 1, d in {32, 64, 128}, dtype in swa_dtype;
 *   B * Hkv * min(n, W) * d * element size / 16 < 2^31 (SWA_ERR_UNSUPPORTED).
 */
int swa_cache_append_chunk(void* k_ring, void* v_ring, const int32_t* pos, const void* k,
                           const void* v, int B, int n, int Hkv, int W, int d, int dtype,
                           void* stream);

/*
 * swa_prefill_chunk - causal windowed attention for a chunk of n new tokens
 * per sequence that continues a sequence whose earlier tokens are in the ring
 * cache (chunked prefill).
 *
 * Token i of sequence b sits at position P = pos[b] + i and attends the
 * positions [max(0, P-W+1), P] (robocikowo definition paragraph; Ultralytics
 * mask 0 <= i-j < w): the positions before pos[b] from ring slot p' mod W
 * (Ultralytics ring-buffer paragraph), the others from the chunk's own rows.
 * The output equals rows pos[b] .. pos[b]+n-1 of swa_prefill (causal, same W)
 * over the whole sequence, provided every earlier position was appended.
 * The ring is only read: append the chunk with swa_cache_append_chunk after
 * this call (same stream), because its tokens overwrite slots that the
 * chunk's early rows still read.  A sequence with pos[b] < 0 gets all-zero
 * output rows.  Positions must stay below 2^31.
 *
 *   q               input [B, Hq, n, d].
 *   k, v            input [B, Hkv, n, d], the chunk's own keys and values.
 *   k_ring, v_ring  input [B, Hkv, W, d], holding positions
 *                   [max(0, pos[b]-W), pos[b]-1].
 *   pos             device int32 [B], the position of each chunk's first token
 *                   (the number of tokens appended before it).
 *   out             output [B, Hq, n, d] (may not alias any input).
 *   B, n, W, Hq, Hkv >= 1, Hq % Hkv == 0, d in {32, 64, 128}, |scale| <= 1024,
 *   dtype in swa_dtype, W * d * element size < 2^31, n <= 2^29 (SWA_ERR_UNSUPPORTED).
 */
int swa_prefill_chunk(const void* q, const void* k, const void* v, const void* k_ring,
                      const void* v_ring, const int32_t* pos, void* out, int B, int n, int W,
                      int Hq, int Hkv, int d, float scale, int dtype, void* stream);

/* Workspace bytes swa_prefill_global needs for these sizes (Hq with the batch
 * folded in; 0 for invalid sizes or G = 0). */
size_t swa_prefill_global_workspace_bytes(int T, int Hq, int G, int d);

/*
 * swa_decode_sinks - swa_decode with attention sinks kept beside the ring.
 *
 * Ultralytics glossary, terms section ("Pozzi di attenzione"): the first
 * tokens of a sequence absorb excess attention weight, and StreamingLLM keeps
 * them in the cache beside the window.  The query at position p = pos[b]
 * attends to the positions {0, ..., min(n_sink-1, p)} together with its
 * window [max(0, p-W+1), p], each position once: window positions from the
 * ring (slot p' mod W), the sink positions before the window from
 * k_sink / v_sink.  Equals row p of swa_prefill_global (causal, global
 * positions 0 .. n_sink-1) when n_sink <= W.  n_sink = 0 is swa_decode.
 *
 *   Arguments, layouts and errors as swa_decode, plus
 *   k_sink, v_sink  input [B, Hkv, n_sink, d]: row s holds the key / value of
 *                   position s (copied from the prompt's K/V by the caller).
 *                   May be NULL when n_sink = 0.
 *   n_sink >= 0.
 *   workspace       at least swa_decode_sinks_workspace_bytes(B, Hq, W, d)
 *                   bytes (n_sink > 0).
 */
int swa_decode_sinks(const void* q, const void* k_ring, const void* v_ring, const void* k_sink,
                     const void* v_sink, int n_sink, const int32_t* pos, void* out, int B, int Hq,
                     int Hkv, int W, int d, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Workspace bytes swa_decode_sinks needs for these sizes (0 for invalid
 * sizes). */
size_t swa_decode_sinks_workspace_bytes(int B, int Hq, int W, int d);

/* Workspace bytes swa_decode needs for these sizes (0 for invalid sizes). */
size_t swa_decode_workspace_bytes(int B, int Hq, int W, int d);

/* Static, human-readable text for a swa_status value. */
const char* swa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
