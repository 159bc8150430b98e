/*
 * attn.h - C ABI of the MI355X (gfx950) causal-attention library (libattn_gfx950.so).
 *
 * What the library computes (sources cited by page title and section):
 *   out = softmax(scale * Q K^T + M) V            per (batch, query head)
 *   "Transformer 架构快速入门" §4.2-4.5 (scores, 1/sqrt(D_h) scale, causal mask, weighted sum of V)
 *   "2.7 Transformer Decoder Block完整解析" §3 (additive -inf causal mask, skipped by index in tiles)
 *   "Transformer 架构快速入门" §6 (MHA / GQA / MQA: query head h reads KV head h / (N_h / N_kv))
 *   "2.7 ..." §4 and "Transformer 架构快速入门" §8 (RoPE on Q and K only)
 *   "Transformer 架构完全深度解析" §九 and "Transformer 架构快速入门" §13.2 (KV-cache decode)
 *   "Transformer 与 LLM：结构、实现与算量" slide 06 (MLA absorbed decode: MQA with one 576-dim row)
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library allocates nothing
 *     and keeps no state between calls; concurrent calls on different streams are safe as long
 *     as they use different workspaces.
 *   - Layouts are row-major. Prefill tensors are BSHD: element (b, s, h, d) of a [B, S, N, D]
 *     tensor sits at ((b * S + s) * N + h) * D + d.
 *   - dtype: ATTN_BF16 means bf16 storage for every floating tensor argument with fp32
 *     accumulation inside; ATTN_F32 means fp32 storage and fp32 arithmetic.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL selects the null stream).
 *     Arguments are validated on the host BEFORE any launch; on an error nothing is launched
 *     and no output is touched. Launch failures are reported as ATTN_ERR_HIP. Faults inside a
 *     kernel surface at the caller's next synchronisation, as for any HIP kernel.
 *   - Tensor pointers must be 16-byte aligned (ATTN_ERR_INVALID otherwise); rope_apply and
 *     attn_kv_append only need element alignment.
 *   - No C++ exception crosses this interface.
 */
#ifndef ATTN_GFX950_H
#define ATTN_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,      /* bad pointer, size, alignment or argument combination */
  ATTN_ERR_UNSUPPORTED = 2,  /* valid request outside the built kernel set (head dim, dtype, ...) */
  ATTN_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_bytes figure */
  ATTN_ERR_HIP = 4           /* the HIP runtime rejected a launch */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Human-readable name of a status code (static storage). */
const char* attn_status_str(int status);

/* ------------------------------------------------------------------------------------------
 * Prefill: causal (or full) self-attention over whole sequences, with optional RoPE.
 *   "Transformer 架构快速入门" §4 (one head), §6.3 (GQA sharing); "2.7 ..." §3.3 (tile skipping).
 *
 * q   [B, S, Nh,  Dh]  read only
 * k   [B, S, Nkv, Dh]  read only (never modified: rotated keys go to the workspace)
 * v   [B, S, Nkv, Dh]  read only
 * out [B, S, Nh,  Dh]  written
 * Nh % Nkv == 0; query head h uses KV head h / (Nh / Nkv).
 * rope_theta > 0 rotates q and k (half-split pairs (i, i + Dh/2), frequency
 *   rope_theta^(-2i/Dh), i = 0-based, angle = position * frequency evaluated in fp64,
 *   positions 0 .. S-1 of each sequence); rope_theta <= 0 uses q and k as given.
 * causal != 0 masks key j for query i when j > i; causal == 0 is full attention.
 * scale <= 0 selects 1 / sqrt(Dh).
 * Supported: ATTN_BF16 with Dh in {64, 128}; ATTN_F32 with Dh in {16, 32, 64}.
 * B == 0 or S == 0 is a valid empty call (nothing launched).
 * workspace: device buffer of attn_prefill_workspace_bytes(...) bytes. With RoPE its leading part
 *   (the angle table and the rotated keys) is required: a smaller or NULL workspace is
 *   ATTN_ERR_WORKSPACE. For ATTN_BF16 the figure ends with 512 bytes of work-list counters, which
 *   are optional: with them, XCDs that run faster take q-tiles left in the slower XCDs' lists;
 *   without them (a workspace just short of the figure, or NULL without RoPE) every q-tile has a
 *   fixed work-group. The output is the same bits either way. The contents are scratch, set by
 *   the call where it needs them; the workspace must not be used by another call until this one
 *   has completed on `stream`.
 * ------------------------------------------------------------------------------------------ */
size_t attn_prefill_workspace_bytes(int B, int S, int Nkv, int Dh, float rope_theta, int dtype);

int attn_prefill(const void* q, const void* k, const void* v, void* out,
                 int B, int S, int Nh, int Nkv, int Dh,
                 float rope_theta, int causal, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * MLA prefill, non-absorbed: "Transformer 与 LLM：结构、实现与算量" slide 06 (prefill keeps W_UK / W_UV
 * un-absorbed: per head, q and k are [128 latent-projected dims ; 64 decoupled RoPE dims] and v is
 * 128 dims; scores use 1/sqrt(192)). Causal self-attention with Dqk = 192 != Dv = 128.
 *
 * q   [B, S, Nh,  192]  read only (q^C ; q^R)
 * k   [B, S, Nkv, 192]  read only (k^C ; k^R; the shared k^R is repeated per KV head)
 * v   [B, S, Nkv, 128]  read only
 * out [B, S, Nh,  128]  written
 * rope_theta > 0 rotates only dims 128..191 of q and k (the decoupled block; half-split pairs
 *   (128 + i, 160 + i), frequency rope_theta^(-2i/64), positions 0 .. S-1); the rotated keys go
 *   to the workspace. causal as attn_prefill; scale <= 0 selects 1 / sqrt(192).
 * Supported: bf16 storage (fp32 accumulation), Nh % Nkv == 0.
 * B == 0 or S == 0 is a valid empty call (nothing launched).
 * workspace: attn_prefill_mla_workspace_bytes(...) bytes. With RoPE its leading part, the angle
 *   table and the keys with their rotated k^R block (k itself is never modified), is required;
 *   the last 512 bytes are optional work-list counters, as for attn_prefill (same bits either way).
 * ------------------------------------------------------------------------------------------ */
size_t attn_prefill_mla_workspace_bytes(int B, int S, int Nkv, float rope_theta);

int attn_prefill_mla(const void* q, const void* k, const void* v, void* out, int B, int S, int Nh, int Nkv,
                     float rope_theta, int causal, float scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------------------------------------------
 * Prefill with a KV cache (chunked prefill): S new query tokens of each sequence attend to the
 * cached keys, their own included. "Transformer 架构完全深度解析" §九 (new K/V are appended to
 * the cache, then the new queries attend to all of it); "Transformer 与 LLM：结构、实现与算量"
 * slide 07 (a long prompt is prefilled in chunks so one request does not hold the GPU).
 *
 * q        [B, S, Nh, Dh]                    read only; query s of sequence b has absolute
 *          position q_start[b] + s
 * kcache   element (b, t, g, d) at ((b * max_ctx + t) * Nkv + g) * ld + d    (ld = row pitch)
 * vcache   same layout and pitch as kcache; rows 0 .. q_start[b] + S - 1 must hold the
 *          sequence's keys/values, already rotated when RoPE is used (attn_kv_append does both)
 * q_start  device int32 [B]: tokens already in the cache before this chunk. A value outside
 *          [0, max_ctx - S] is clamped into it for memory safety (the result is then not
 *          meaningful).
 * out      [B, S, Nh, Dh]                    written
 * causal != 0: the query at position p attends keys 0 .. p (the square causal mask shifted so
 *          that the chunk's last query sees the last key); causal == 0: all q_start[b] + S keys.
 * window > 0 (causal only): sliding window, the query at position p attends keys
 *          max(0, p - window + 1) .. p, plus the first `sinks` keys 0 .. sinks-1 (attention sinks)
 *          - "Transformer 与 LLM：结构、实现与算量" slide 07 (window W, e.g. 4096; sink = the first 4
 *          tokens kept). window == 0: no window (sinks must be 0). Tiles outside every row's window
 *          and past the sinks are neither loaded nor computed.
 * rope_theta > 0 rotates q at its absolute position; the cached keys are used as stored. The
 *          rotary span is the leading rope_dims dims (0 selects Dh; a multiple of 32), frequencies
 *          rope_theta^(-2i/rope_dims), pairs (i, i + rope_dims/2), or (2i, 2i + 1) with
 *          rope_interleaved != 0 - "Transformer 架构快速入门" §8.1-8.2 (either pairing; D_r may be
 *          a part of the head). It must match the rotation the cached keys received.
 *          scale <= 0 selects 1 / sqrt(Dh).
 * Supported: ATTN_BF16, Dh in {64, 128}, 1 <= S <= max_ctx, ld % 8 == 0, ld >= Dh.
 * workspace: attn_prefill_cached_workspace_bytes(...) bytes: the RoPE angle table (required with
 *   RoPE), then 512 bytes of optional work-list counters, as for attn_prefill (same bits either way).
 * With q_start[b] = 0 and S = max_ctx this is exactly attn_prefill on the cached keys.
 * ------------------------------------------------------------------------------------------ */
size_t attn_prefill_cached_workspace_bytes(int max_ctx, int Dh, float rope_theta);

int attn_prefill_cached(const void* q, const void* kcache, const void* vcache, const int32_t* q_start,
                        void* out, int B, int S, int Nh, int Nkv, int Dh, int max_ctx, long long ld,
                        float rope_theta, int rope_dims, int rope_interleaved, int causal, int window,
                        int sinks, float scale, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ------------------------------------------------------------------------------------------
 * KV-cache append with RoPE fused: writes S new tokens of each sequence into the caches at rows
 * start[b] .. start[b] + S - 1, rotating K at those absolute positions.
 *   "Transformer 架构完全深度解析" §九 (concat of the new K/V to the cache), "2.7 ..." §4 and
 *   "Transformer 架构快速入门" §8.2-8.3 (RoPE on K: frequency theta^(-2i/Dh), fp64 angle,
 *   cos/sin rounded once to fp32, rotation in fp32, one rounding to bf16).
 *
 * k_new, v_new [B, S, Nkv, Dh]  read only
 * kcache, vcache: layout of attn_prefill_cached / attn_decode (pitches ldk, ldv), written only
 *          at the appended rows. start: device int32 [B], clamped to [0, max_ctx - S].
 * rope_theta > 0 rotates the leading rope_dims dims of K (0 selects Dh; even), frequencies
 *          rope_theta^(-2i/rope_dims), pairs (i, i + rope_dims/2), or (2i, 2i + 1) with
 *          interleaved != 0; the other dims are copied. rope_theta <= 0 copies K unchanged.
 *          V is copied unchanged.
 * Supported: ATTN_BF16, Dh % 8 == 0 and Dh <= 1024, 1 <= S <= max_ctx. With every pointer
 *          16-byte aligned and ldk, ldv multiples of 8 the rows move as 16-byte vectors, otherwise
 *          element by element; both give the same bits.
 * A key appended here and a key rotated by attn_prefill's RoPE step carry identical bits.
 * ------------------------------------------------------------------------------------------ */
int attn_kv_append(const void* k_new, const void* v_new, void* kcache, void* vcache, const int32_t* start,
                   int B, int S, int Nkv, int Dh, int max_ctx, long long ldk, long long ldv,
                   float rope_theta, int rope_dims, int interleaved, int dtype, void* stream);

/* ------------------------------------------------------------------------------------------
 * KV-cache decode: one new query token per sequence attends to every cached key of its head.
 *   "Transformer 架构完全深度解析" §九 (append new K/V, then attend the new query to the cache),
 *   "Transformer 与 LLM：结构、实现与算量" slide 06 (absorbed MLA = MQA over one shared row).
 *
 * q        [B, Nh, Dqk]                      read only
 * kcache   element (b, t, g, d) at ((b * max_ctx + t) * Nkv + g) * ldk + d,  d < Dqk
 * vcache   element (b, t, g, d) at ((b * max_ctx + t) * Nkv + g) * ldv + d,  d < Dv
 *          vcache MAY equal kcache (MLA: V is the first Dv elements of the cached K row).
 * ctx_lens device int32 [B]: keys 0 .. ctx_lens[b]-1 are attended, the new token's own key
 *          included (it is appended before the call). Values must lie in [1, max_ctx]; a value
 *          outside is clamped to [0, max_ctx] for memory safety and 0 keys give an all-zero
 *          output row (the result is then not meaningful).
 * out      [B, Nh, Dv]                      written
 * rope_theta > 0 rotates q at position ctx_lens[b]-1 (the cache holds already-rotated keys):
 *          half-split pairs over all Dqk dims for Dqk == Dv; for the MLA form only the decoupled
 *          q^R block, dims 512..575 (pairs (512 + i, 544 + i), frequency rope_theta^(-2i/64)) -
 *          "Transformer 与 LLM：结构、实现与算量" slide 06. scale <= 0 selects 1 / sqrt(Dqk).
 * Supported (ATTN_BF16 only): Dqk == Dv in {64, 128} with Nh % Nkv == 0 and a group size
 *   G = Nh / Nkv of at most 16 or a multiple of 16 (query heads are processed 16 at a time);
 *   and the MLA form Dqk = 576, Dv = 512, Nkv = 1, vcache == kcache, ldv == ldk, Nh % 16 == 0.
 * workspace: at least attn_decode_workspace_bytes(...) bytes (split-KV partial results); may be
 *   NULL when that figure is 0 (the MLA form when every sequence fits one chunk: the kernel then
 *   writes the output directly).
 * ------------------------------------------------------------------------------------------ */
size_t attn_decode_workspace_bytes(int B, int Nh, int Nkv, int Dqk, int Dv, int max_ctx, int dtype);

int attn_decode(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens,
                void* out, int B, int Nh, int Nkv, int Dqk, int Dv, int max_ctx,
                long long ldk, long long ldv, float rope_theta, float scale, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * KV-cache decode that allocates nothing, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, layouts, supported shapes and results are those of attn_decode, which it calls
 * (same kernels, same bits); only the workspace is gone. The split-KV partials go to a static
 * device buffer of attn_decode_noalloc_max_bytes() bytes (64 MiB) inside the library, one per GPU,
 * held from its first use on that GPU until the process ends. No hipMalloc, hipFree or other
 * allocating call is made.
 * Errors: ATTN_ERR_WORKSPACE when attn_decode_workspace_bytes(...) of the call exceeds that size
 *          (nothing is launched); otherwise as attn_decode.
 * Concurrency: every call on one GPU uses that GPU's one buffer. Calls that overlap in time on
 *          one GPU (different streams, or host threads without ordering) race and give wrong
 *          results; calls ordered on one stream are safe. The buffer keeps the last call's
 *          partials; nothing in it needs clearing (each call writes every partial it reads).
 * ------------------------------------------------------------------------------------------ */
size_t attn_decode_noalloc_max_bytes(void);

int attn_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens,
                        void* out, int B, int Nh, int Nkv, int Dqk, int Dv, int max_ctx,
                        long long ldk, long long ldv, float rope_theta, float scale, int dtype,
                        void* stream);

/* ------------------------------------------------------------------------------------------
 * RoPE, in place: rotate every head vector of x [B, S, N, Dh] by its position.
 *   "2.7 ..." §4 (half-split pairs), "Transformer 架构快速入门" §8.2-8.3 (frequencies, adjacent
 *   pairs), "Transformer 架构完全深度解析" §七.
 * positions: device int32 [B * S] (position of token (b, s) at b * S + s), or NULL for s.
 * interleaved == 0: pairs (i, i + Dh/2); interleaved != 0: pairs (2i, 2i + 1).
 * Frequency theta^(-2i/Dh), i = 0 .. Dh/2 - 1; angle = position * frequency in fp64.
 * Supported: ATTN_F32 and ATTN_BF16, Dh even and <= 1024, theta > 0.
 * ------------------------------------------------------------------------------------------ */
int rope_apply(void* x, const int32_t* positions, int B, int S, int N, int Dh,
               float theta, int interleaved, int dtype, void* stream);

/* ------------------------------------------------------------------------------------------
 * Profiling: time the main kernel of a call apart from its helper launches (the RoPE table and
 * key rotation of attn_prefill, the span pass of attn_prefill_mla, the split reduction of
 * attn_decode). After attn_set_kernel_events(before, after), every attn_prefill,
 * attn_prefill_cached, attn_prefill_mla and attn_decode call made by the SAME host thread records
 * the HIP event `before` on its stream right before the attention kernel's launch and `after`
 * right after it (the decode's split kernel); hipEventElapsedTime(before, after) is then that
 * kernel's duration. The events are owned by the caller (hipEvent_t, created with timing
 * enabled). attn_set_kernel_events(NULL, NULL) stops the recording.
 * Errors: ATTN_ERR_INVALID if exactly one of the two is NULL; a failed record makes the call
 *          return ATTN_ERR_HIP.
 * ------------------------------------------------------------------------------------------ */
int attn_set_kernel_events(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GFX950_H */
