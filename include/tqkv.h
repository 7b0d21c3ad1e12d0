/*
 * tqkv.h -- C ABI of libtqkv.so: TurboQuant KV-cache store and speculative
 * verification attention for AMD Instinct MI355X (gfx950).
 *
 * The two calls follow the problem statement of "Speculative decoding on
 * Intel Arc: TurboQuant KV + a fused N_spec kernel" (turboquant-xpu blog,
 * 2026-04-14):
 *   - tqkv_store  is the fused store (Context section: Walsh-Hadamard
 *     rotation + Lloyd-Max codebook for keys, uniform scalar quantisation for
 *     values, 3-4 bits per coordinate; the k8v4 preset keeps FP8 keys,
 *     Part 6);
 *   - tqkv_verify is the fused N_spec verification attention of Part 3
 *     (query [N_spec, B, Hq, D] -> output of the same shape) with the causal
 *     window of Part 4 (query n attends to cached_len + n + 1 tokens) and the
 *     split-KV partition + log-sum-exp reduction of Part 2.
 *
 * Memory and streams.  Every pointer argument is device memory owned by the
 * caller, except the tqkv_cache descriptor itself (host memory, read during
 * the call only).  The library allocates nothing on the device, copies
 * nothing between host and device, and never synchronises: each call
 * enqueues its kernels on `stream` (a hipStream_t; NULL = the default
 * stream) and returns.  Calls are reentrant; the library keeps no state
 * besides read-only constant tables, the per-device values it looks up once
 * (compute-unit count) and the scratch array of tqkv_verify_noalloc (a
 * static device array of TQKV_NOALLOC_SCRATCH_BYTES per device, which only
 * that call uses).
 *
 * Errors.  Every entry point validates its host-side arguments first and
 * returns a negative tqkv_status without launching anything when they are
 * invalid.  TQKV_ERR_LAUNCH reports a failed kernel launch (hipGetLastError).
 * Device-side values (seq_idx, pos, seq_lens) cannot be checked on the host
 * without a synchronisation; the kernels clamp or skip out-of-range values so
 * that no access leaves the caller's buffers, and the documented
 * preconditions say what the result then is.
 *
 * Cache layout (all sizes for D = 128).  Per (sequence b, KV head hk) the
 * tokens are cut into blocks of 16; block blk of (b, hk) starts at
 *   base + ((b * Hk + hk) * nblk + blk) * tqkv_block_bytes(preset),
 * nblk = ceil(max_seq / 16).  A k3v4_nc block is 1920 B (120 B per token:
 * 48 B of 3-bit key codes, 64 B of 4-bit value codes, fp16 norm, fp16 norm
 * correction, fp16 value scale, fp16 value zero); a k4v4_nc block is 2176 B
 * (136 B per token: 64 B of 4-bit key codes, then the same fields as
 * k3v4_nc); a k8v4 block is 3168 B (198 B per token: 128 B of FP8 E4M3 key
 * codes, 64 B of value codes, fp16 key scale, value scale, value zero).  The exact byte and bit placement is
 * given by the byte offsets in the library source (common.h); the stored
 * bytes of a token depend only on that token's K and V.
 *
 * Paged cache (tqkv_paged_cache).  The cache the pages measure is a pool of
 * blocks of 16 tokens, each holding those tokens for every KV head ("Roofline"
 * of Part 2: blocks x 16 tokens x Hk x slot bytes).  Here a page is exactly
 * that: page p of the pool holds Hk of the 16-token blocks above, head hk's
 * block at base + (p * Hk + hk) * tqkv_block_bytes(preset), byte-identical to
 * the block a contiguous cache holds for the same 16 tokens.  A block table
 * maps the 16-token run j of sequence b (tokens [16 j, 16 j + 16)) to its
 * page, in the manner of a paged serving engine; the store addresses tokens
 * by slot = page * 16 + position in the page.
 */
#ifndef TQKV_H
#define TQKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQKV_HEAD_DIM 128    /* the only supported head size */
#define TQKV_BLOCK_TOKENS 16 /* tokens per cache block */
#define TQKV_MAX_QLEN 128    /* queries per sequence (n_spec, or the largest ragged count) */
#define TQKV_MAX_ROWS 8192   /* (Hq / Hk) * queries per sequence must not exceed this */
#define TQKV_MAX_PAGES_PER_SEQ 524288 /* block-table row length of a paged cache (8M tokens) */
#define TQKV_NOALLOC_SCRATCH_BYTES (8u << 20) /* workspace held by the library per device for tqkv_verify_noalloc */

typedef enum {
    TQKV_K8V4 = 1,    /* FP8 E4M3 keys with a per-token fp16 scale, 4-bit values */
    TQKV_K3V4_NC = 2, /* WHT-rotated 3-bit Lloyd-Max keys + norm correction, 4-bit values */
    TQKV_K4V4_NC = 3  /* the same with 4-bit (16-level) Lloyd-Max keys */
} tqkv_preset;

typedef enum {
    TQKV_Q_F32 = 0,
    TQKV_Q_F16 = 1
} tqkv_qtype;

typedef enum {
    TQKV_OK = 0,
    TQKV_ERR_ARG = -1,         /* a null pointer, a negative size, a bad enum */
    TQKV_ERR_UNSUPPORTED = -2, /* D != 128, too many rows per KV head, Hq % Hk != 0 */
    TQKV_ERR_ALIGN = -3,       /* a device pointer is not aligned as documented */
    TQKV_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    TQKV_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch */
    TQKV_ERR_DEVICE = -6       /* no usable gfx950 device is current */
} tqkv_status;

/* A quantised KV cache in caller-owned device memory of
 * tqkv_cache_bytes(preset, B, Hk, D, max_seq) bytes, 16-byte aligned. */
typedef struct tqkv_cache {
    int32_t preset;  /* tqkv_preset */
    int32_t B;       /* sequences */
    int32_t Hk;      /* KV heads */
    int32_t D;       /* head size, must be 128 */
    int32_t max_seq; /* token capacity per sequence */
    void *base;      /* device pointer */
} tqkv_cache;

/* A paged quantised KV cache: a pool of num_pages pages in caller-owned
 * device memory of tqkv_paged_cache_bytes(preset, Hk, D, num_pages) bytes,
 * 16-byte aligned, and (for the verify calls) the block table of a batch of
 * B sequences.  The stores need only the pool fields. */
typedef struct tqkv_paged_cache {
    int32_t preset;             /* tqkv_preset */
    int32_t Hk;                 /* KV heads */
    int32_t D;                  /* head size, must be 128 */
    int32_t num_pages;          /* pages in the pool, at most 2^27 - 1 */
    void *base;                 /* device pointer to the pool */
    const int32_t *block_table; /* device int32 [B, max_pages], 4-byte aligned: page of
                                   tokens [16 j, 16 j + 16) of sequence b at
                                   block_table[b * max_pages + j] */
    int32_t B;                  /* sequences of the batch */
    int32_t max_pages;          /* row length of the block table: token capacity
                                   16 * max_pages per sequence, <= TQKV_MAX_PAGES_PER_SEQ */
} tqkv_paged_cache;

/* Bytes per token and KV head ("slot"): 120 (k3v4_nc), 136 (k4v4_nc) or
 * 198 (k8v4); 0 for a bad preset.  The pages size the cache per token and
 * KV head ("Speculative decoding on Intel Arc", Part 2, Roofline: a k8v4
 * slot of 196 B); k8v4 here also keeps the per-token fp16 key scale (+2 B),
 * and the 3-bit preset packs 128 codes into 48 B next to the same 4-bit
 * values (Context: 3-4 bits per coordinate). */
size_t tqkv_slot_bytes(int preset);

/* Bytes per 16-token block: 16 * tqkv_slot_bytes(preset) (the 16-token
 * block is the unit of the pages' paged cache, Part 2, Roofline). */
size_t tqkv_block_bytes(int preset);

/* Bytes of a whole contiguous cache, B * Hk * ceil(max_seq / 16) blocks (the
 * Roofline count of Part 2: blocks x 16 tokens x Hk x slot); 0 for invalid
 * arguments. */
size_t tqkv_cache_bytes(int preset, int B, int Hk, int D, int max_seq);

/* Bytes of a paged pool of num_pages pages: num_pages * Hk * tqkv_block_bytes(preset);
 * 0 for invalid arguments. */
size_t tqkv_paged_cache_bytes(int preset, int Hk, int D, int num_pages);

/* store(K, V, codes): quantise T new tokens for all Hk heads into the cache.
 *   K, V     device, fp16 [T, Hk, 128] (row-major), 2-byte aligned
 *   seq_idx  device, int32 [T]: sequence of token t, in [0, B)
 *   pos      device, int32 [T]: position of token t, in [0, max_seq)
 * Keys (k3v4_nc, k4v4_nc): fp32 norm n, normalised Sylvester WHT of k/n, a
 * 3-bit (4-bit) code per coordinate against the 8 (16) N(0, 1/128)
 * Lloyd-Max levels, norm correction gamma = 1/||c[codes]||, fp16 n and
 * gamma.  Keys (k8v4): scale
 * s = fp16(max|k| / 448), codes = e4m3(k / s) rounded to nearest even and
 * saturated.  Values: zero = min v, scale = fp16((max v - min v) / 15),
 * code = clamp(rint((v - zero) / scale), 0, 15).  The bytes written are
 * bit-identical to the specification (all arithmetic IEEE binary32, RNE).
 * (seq_idx, pos) pairs must be distinct within one call; an entry out of
 * range is skipped (nothing written).  T == 0 is a no-op; T rounded up to a
 * multiple of 16, times Hk, must not exceed 2^31 - 1 (TQKV_ERR_UNSUPPORTED).
 * Returns TQKV_OK or a negative tqkv_status. */
int tqkv_store(const tqkv_cache *cache, const void *K, const void *V, const int32_t *seq_idx,
               const int32_t *pos, int T, void *stream);

/* tqkv_store into a paged pool (block_table, B and max_pages are not used):
 *   slot_mapping  device, int32 [T], 4-byte aligned: token t goes to
 *                 position slot % 16 of page slot / 16; a negative slot
 *                 (padding) or a page >= num_pages is skipped
 * The bytes written for a token are those tqkv_store writes for it.  Slots
 * must be distinct within one call.  T == 0 is a no-op.
 * Returns TQKV_OK or a negative tqkv_status. */
int tqkv_paged_store(const tqkv_paged_cache *cache, const void *K, const void *V, const int32_t *slot_mapping,
                     int T, void *stream);

/* Number of key-range partitions tqkv_verify uses for num_splits (0 = auto)
 * on this cache and shape; 0 for invalid arguments.  The partitions are the
 * first stage of the pages' two-stage split-KV decode ("Speculative
 * decoding on Intel Arc", Part 2: NUM_KV_SPLITS ranges per (b, hk), merged
 * by log-sum-exp in stage 2). */
int tqkv_verify_num_splits(const tqkv_cache *cache, int n_spec, int Hq, int num_splits);

/* Device workspace tqkv_verify needs, returned through *bytes: when more
 * than one key range is used, the partial softmax states of every range
 * (the stage-1 outputs of Part 2's split-KV decode: per row and range a
 * running max, a sum and a binary16 partial output; 0 bytes otherwise).
 * The size comes back through a pointer so that the return value can
 * report an invalid shape or a missing device as a status.
 * Returns TQKV_OK or a negative tqkv_status. */
int tqkv_verify_workspace_bytes(const tqkv_cache *cache, int n_spec, int Hq, int num_splits,
                                size_t *bytes);

/* verify(Q, cache, lens): attention of n_spec speculative queries per
 * sequence over the quantised cache.
 *   Q         device, [n_spec, B, Hq, 128] of q_dtype, 16-byte aligned;
 *             1 <= n_spec <= TQKV_MAX_QLEN, (Hq / Hk) * n_spec <= TQKV_MAX_ROWS
 *   seq_lens  device, int32 [B]: tokens in the cache for sequence b, the
 *             n_spec speculative ones included (cached_len = seq_lens[b] - n_spec)
 *   causal    1: query n attends to tokens [0, cached_len + n + 1);
 *             0: every query attends to tokens [0, seq_lens[b])
 *   num_splits  key-range partitions per (b, hk), 0 = auto; at most
 *             min(1024, ceil(ceil(max_seq / 32) / 4)) are used (one range
 *             covers at least four 32-token tiles); tqkv_verify_num_splits
 *             returns the count a call will use
 *   sm_scale  softmax scale, 0 = 1/sqrt(128)
 *   out       device, fp32 [n_spec, B, Hq, 128], 16-byte aligned
 *   workspace device, 256-byte aligned, >= tqkv_verify_workspace_bytes(...)
 *             (may be NULL when that is 0); its contents on entry do not
 *             matter and are overwritten
 * Query head hq reads KV head hq / (Hq / Hk).  k3v4_nc and k4v4_nc queries
 * are rotated by the same normalised WHT as the keys.  Preconditions (device values):
 * n_spec <= seq_lens[b] <= max_seq and every token below seq_lens[b] was
 * stored; a larger seq_lens[b] is clamped to max_seq, and a row that sees no
 * token is NaN.  The result matches plain softmax attention over the
 * dequantised cache up to fp16 rounding of the MFMA operands.
 * Returns TQKV_OK or a negative tqkv_status. */
int tqkv_verify(const tqkv_cache *cache, const void *Q, int q_dtype, const int32_t *seq_lens,
                int n_spec, int Hq, int causal, int num_splits, float sm_scale, float *out,
                void *workspace, size_t workspace_bytes, void *stream);

/* tqkv_verify for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, result, preconditions and errors as tqkv_verify, but
 * the workspace is the library's own scratch array of
 * TQKV_NOALLOC_SCRATCH_BYTES per device (a static device array, created
 * when the library's code is loaded on a device and held until the process
 * ends).  The call allocates and frees nothing.  A shape whose
 * tqkv_verify_workspace_bytes exceeds TQKV_NOALLOC_SCRATCH_BYTES returns
 * TQKV_ERR_WORKSPACE without launching (with 64 query rows per KV head
 * every (b, hk, key range) takes 16896 bytes: 8 MiB holds
 * B * Hk * splits <= 496, e.g. the PoC shape's 16 * 16).  Every call on a device shares that
 * device's array and nothing in it needs clearing (each call writes the
 * partial states before it reads them); calls that may overlap on one device
 * (several streams, several host threads) race on it and must be ordered
 * by the caller, e.g. issued on one stream.
 * Returns TQKV_OK or a negative tqkv_status. */
int tqkv_verify_noalloc(const tqkv_cache *cache, const void *Q, int q_dtype, const int32_t *seq_lens,
                        int n_spec, int Hq, int causal, int num_splits, float sm_scale, float *out,
                        void *stream);

/* tqkv_verify with a different number of queries per sequence, packed (the
 * verify of per-sequence draft lengths, or a continuation chunk of up to
 * TQKV_MAX_QLEN tokens; the integration path of the pages' Part 6):
 *   cu_q      device, int32 [B + 1], 4-byte aligned: sequence b owns query
 *             rows [cu_q[b], cu_q[b + 1]) of Q and out, q_b = their count;
 *             its queries are its last q_b tokens (cached_len = seq_lens[b] - q_b)
 *   max_q     host: an upper bound of every q_b, 1 <= max_q <= TQKV_MAX_QLEN;
 *             counts above it are cut to max_q; the workspace and split
 *             count are those of tqkv_verify with n_spec = max_q
 *   Q         device, [cu_q[B], Hq, 128] of q_dtype, 16-byte aligned
 *   out       device, fp32 [cu_q[B], Hq, 128], 16-byte aligned
 * Query n of sequence b attends to tokens [0, cached_len + n + 1) (causal)
 * or [0, seq_lens[b]).  Rows of out that no sequence owns are not written.
 * Returns TQKV_OK or a negative tqkv_status. */
int tqkv_verify_varlen(const tqkv_cache *cache, const void *Q, int q_dtype, const int32_t *cu_q, int max_q,
                       const int32_t *seq_lens, int Hq, int causal, int num_splits, float sm_scale, float *out,
                       void *workspace, size_t workspace_bytes, void *stream);

/* store + verify in one launch, for the speculative-decode step of the
 * pages' Part 4 (the N_spec draft tokens are written to the cache, then
 * their queries attend to it):
 *   K, V      device, fp16 [n_spec, B, Hk, 128], 2-byte aligned: token n of
 *             sequence b is quantised into position seq_lens[b] - n_spec + n
 *             (exactly the bytes tqkv_store writes for it)
 *   the other arguments and the result are those of tqkv_verify.
 * Equivalent to tqkv_store of those n_spec * B tokens followed by
 * tqkv_verify; for small steps (n_spec * ceil(Hq / Hk * n_spec / 32) <= 32)
 * without the separate store launch: the work-groups that read the new
 * tokens' tiles quantise them first.  Same preconditions as tqkv_verify,
 * plus n_spec <= seq_lens[b].
 * Returns TQKV_OK or a negative tqkv_status. */
int tqkv_store_verify(const tqkv_cache *cache, const void *K, const void *V, const void *Q, int q_dtype,
                      const int32_t *seq_lens, int n_spec, int Hq, int causal, int num_splits, float sm_scale,
                      float *out, void *workspace, size_t workspace_bytes, void *stream);

/* The verify calls on a paged cache: the same arguments, results and
 * preconditions as tqkv_verify_num_splits, tqkv_verify_workspace_bytes,
 * tqkv_verify, tqkv_verify_varlen and tqkv_store_verify, with every block of
 * sequence b read from (and, for the store, written to) the page the block
 * table names.  Besides, every table entry for tokens below seq_lens[b] must
 * name a page of the pool holding those tokens; an entry outside
 * [0, num_pages) reads page 0 instead (and the fused store skips it), so no
 * access leaves the pool.  The split count is raised where needed so that
 * one work-group covers at most 8192 tokens. */
int tqkv_paged_verify_num_splits(const tqkv_paged_cache *cache, int n_spec, int Hq, int num_splits);
int tqkv_paged_verify_workspace_bytes(const tqkv_paged_cache *cache, int n_spec, int Hq, int num_splits,
                                      size_t *bytes);
int tqkv_paged_verify(const tqkv_paged_cache *cache, const void *Q, int q_dtype, const int32_t *seq_lens,
                      int n_spec, int Hq, int causal, int num_splits, float sm_scale, float *out, void *workspace,
                      size_t workspace_bytes, void *stream);
int tqkv_paged_verify_varlen(const tqkv_paged_cache *cache, const void *Q, int q_dtype, const int32_t *cu_q,
                             int max_q, const int32_t *seq_lens, int Hq, int causal, int num_splits, float sm_scale,
                             float *out, void *workspace, size_t workspace_bytes, void *stream);
int tqkv_paged_store_verify(const tqkv_paged_cache *cache, const void *K, const void *V, const void *Q, int q_dtype,
                            const int32_t *seq_lens, int n_spec, int Hq, int causal, int num_splits, float sm_scale,
                            float *out, void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *tqkv_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int tqkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQKV_H */
