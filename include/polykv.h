/*
 * polykv.h - C ABI of the shared, asymmetrically compressed KV pool and of
 * fused multi-agent decode attention over it, for AMD Instinct MI355X (gfx950).
 *
 * What the pool is (PolyKV explainer, section 2.A "core architecture"):
 * the KV state of a shared context is computed once, compressed, and stored
 * as one object that many agents read; its memory does not grow with the
 * number of agents.  How it is compressed (section 2.B "asymmetric
 * compression scheme"): K becomes int8 under a per-tensor linear scale; V is
 * rotated by a fast Walsh-Hadamard transform, normalised, and each
 * coordinate is replaced by the index of its Lloyd-Max cell for N(0, 1).
 * CoMixKV (news article: abstract and "incremental quantization strategy")
 * chooses the V bit width per (agent, layer) among 2, 3 and 4, keeps the most
 * recent tokens at native precision, and never re-quantises stored blocks.
 *
 * Conventions shared by every entry point:
 *  - Return value: PKV_OK (0) or a negative PKV_E* code.  All validation is
 *    done on the host, synchronously, before anything is enqueued; on error
 *    nothing is enqueued and no output is modified.
 *  - Device memory is always owned by the caller.  The library allocates
 *    neither device nor pinned host memory and keeps no global state except
 *    immutable constant tables.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every device effect is enqueued on it, asynchronously.  Calls that touch
 *    the same pool must be ordered on one stream by the caller; calls on
 *    distinct pools and workspaces may run concurrently.
 *  - Inputs holding NaN or Inf give undefined (but memory-safe) results.
 */
#ifndef POLYKV_H
#define POLYKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_MAX_LAYERS 128

enum {
    PKV_OK = 0,
    PKV_EINVAL = -1,        /* null pointer, bad shape or count, inconsistent arguments */
    PKV_EUNSUPPORTED = -2,  /* head_dim not 64/128, bits not 2/3/4, unknown dtype */
    PKV_ECAPACITY = -3,     /* append would exceed the pool's token capacity */
    PKV_ENOSPACE = -4,      /* device buffer or workspace smaller than required */
    PKV_EHIP = -5           /* a kernel launch failed (hipGetLastError) */
};

/* Element types.  The type is a plain 32-bit integer so that any value a caller passes can be
 * read and rejected (PKV_EUNSUPPORTED); an enum type would not hold values outside its list. */
enum { PKV_F32 = 0, PKV_BF16 = 1 };
typedef int32_t pkv_dtype;

/* Shape of one pool.  K always uses 8 bits; V uses v_bits[l] bits in layer l.
 * v_signs: the V rotation's sign mask, bit i (little-endian over the 16 bytes)
 * set = coordinate i of every V vector negated before the FWHT and the decoded
 * output negated after the inverse FWHT (rotation H D with D = diag(+-1), a
 * randomised-Hadamard variant chosen by the caller); all zero = the plain FWHT
 * of PolyKV explainer, section 2.B.  Bits at or above head_dim must be 0. */
typedef struct {
    int32_t n_layers;                /* 1 .. PKV_MAX_LAYERS */
    int32_t n_kv_heads;              /* >= 1 */
    int32_t head_dim;                /* 64 or 128 */
    int32_t capacity_tokens;         /* >= 1; rounded up to a multiple of 32 internally */
    uint8_t v_bits[PKV_MAX_LAYERS];  /* 2, 3 or 4 for layers 0 .. n_layers-1 */
    uint8_t v_signs[16];             /* rotation sign mask (see above); zero = plain FWHT */
    uint8_t k_scale;                 /* K-scale granularity, PKV_KSCALE_* (0 = per tensor, the pages') */
    uint8_t v_norm;                  /* stored V norm, PKV_VNORM_* (0 = plain ||v||) */
    uint8_t reserved[2];             /* must be 0 */
} pkv_pool_config;

/* Codec variants, measured as ablations (PolyKV explainer, section 2.B names a
 * per-tensor K scale and a per-vector V norm; the QKVShare blog, section 3.2,
 * weighs per-tensor, per-token and per-channel granularity):
 *  PKV_KSCALE_TENSOR   one scale per layer and append block (q8_0 over the block)
 *  PKV_KSCALE_TOKEN    one scale per stored K vector (token, kv head)
 *  PKV_KSCALE_CHANNEL  one scale per (layer, kv head, channel), taken from the
 *                      first append; later appends use it and clamp at +-127
 *  PKV_VNORM_PLAIN     Vn = ||v||
 *  PKV_VNORM_CORRECTED Vn = fl(fl(||v|| * fl(sqrt(d))) / ||c_hat||), ||c_hat|| the
 *                      fp32 norm of the chosen centroids (same halving tree), so
 *                      the decoded vector keeps the input's norm; codes unchanged */
#define PKV_KSCALE_TENSOR 0
#define PKV_KSCALE_TOKEN 1
#define PKV_KSCALE_CHANNEL 2
#define PKV_VNORM_PLAIN 0
#define PKV_VNORM_CORRECTED 1

/*
 * Descriptor of one pool: a plain struct in caller-owned host memory (no
 * destroy call).  It records where each region lives inside the caller's
 * device buffer and how many tokens each layer holds.  The byte layout, each
 * region starting on a 256-byte boundary, with tc = capacity rounded up to 32:
 *
 *   Kq    int8 [L][Hkv][tc][d]            K codes (two's complement, -127..127)
 *   Vn    f32  [L][Hkv][tc]               V norms (||v||, or the corrected norm)
 *   Ks    f32  [L][tc]                    K scale of the append block holding each token
 *              ([L][Hkv][tc] per token, [L][Hkv][d] per channel)
 *   Vmax  f32  [L][Hkv]                   max V norm over the tokens stored so far
 *   Vc    u8   per layer l: [Hkv][tc/8][d * v_bits[l]]   packed V code groups
 *   amax  u32  [L] ([L][Hkv][d] per channel)   scratch used by pool_quantize_append
 *
 * A V code group covers 8 consecutive tokens of one (layer, kv head): for
 * each dimension i = 0 .. d-1 in order, one little-endian field of
 * 8 * bits bits holding the codes of the 8 tokens, token j in bits
 * [bits*j, bits*(j+1)) (at 3 bits: 8 codes in 3 bytes).  Codes index the
 * Lloyd-Max centroids in ascending order.  Bits of tokens not yet stored are 0.
 */
typedef struct {
    pkv_pool_config cfg;
    void* base;                          /* device buffer (caller-owned) */
    uint64_t bytes;                      /* bytes of the buffer in use (= pool_bytes(cfg)) */
    int32_t tc;                          /* capacity rounded up to 32 */
    int32_t n_tokens[PKV_MAX_LAYERS];    /* tokens stored per layer; advanced by appends */
    uint64_t off_kq, off_vn, off_ks, off_vmax, off_amax;
    uint64_t off_vc[PKV_MAX_LAYERS + 1]; /* off_vc[l] .. off_vc[l+1]: codes of layer l */
} pkv_pool;

/*
 * Bytes of device memory one pool of this shape needs (the layout above).
 * The value does not depend on how many agents will read the pool (PolyKV
 * explainer, section 4 "memory efficiency": pool size is constant in the agent
 * count).  Returns 0 if cfg is NULL or invalid.
 */
size_t pool_bytes(const pkv_pool_config* cfg);

/*
 * Lay a pool out in a caller-owned device buffer.  Host-only: writes the
 * descriptor *out (offsets, tc, n_tokens = 0) and enqueues no device work.
 * dev_buf must be 256-byte aligned and dev_bytes >= pool_bytes(cfg).
 * Errors: PKV_EINVAL (NULL, misaligned), PKV_EUNSUPPORTED (head_dim, bits),
 * PKV_ENOSPACE (dev_bytes too small).
 */
int pool_build(const pkv_pool_config* cfg, void* dev_buf, size_t dev_bytes, pkv_pool* out);

/*
 * Quantise n_tokens new tokens into layers [layer_begin, layer_begin +
 * layer_count) of the pool (PolyKV explainer, section 2.B; CoMixKV article,
 * "incremental quantization strategy": new tokens are appended, earlier
 * tokens are never re-quantised).
 *
 *   k, v   device [layer_count][n_kv_heads][n_tokens][head_dim], dtype
 *          PKV_F32 or PKV_BF16, contiguous; read only.
 *
 * Per layer, the K values of this call form one tensor with one scale:
 * s = amax / 127 (amax = max |k| over all heads, tokens and channels of that
 * layer in this call), codes = clamp(rint(k / s), -127, 127), or s = 0 and
 * codes 0 when amax = 0 (PKV_KSCALE_TOKEN: the same rule per K vector;
 * PKV_KSCALE_CHANNEL: per channel over the first append's tokens).  Each V vector x gets n = ||x|| (squares summed by a
 * halving tree, correctly rounded sqrt), z = H x (unnormalised Sylvester
 * Hadamard, butterflies with ascending half-width), y = z * (1/n), and
 * code_i = number of Lloyd-Max N(0, 1) thresholds strictly below y_i; n = 0
 * gives codes 0.  All of it is fp32 without contraction, so codes are
 * reproducible bit for bit.
 *
 * All layers in the range must hold the same number of tokens before the
 * call.  On success pool->n_tokens[l] is advanced on the host at enqueue time.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED (dtype), PKV_ECAPACITY, PKV_EHIP.
 */
int pool_quantize_append(pkv_pool* pool, int32_t layer_begin, int32_t layer_count,
                         const void* k, const void* v, pkv_dtype dtype, int32_t n_tokens,
                         void* stream);

/* Arguments of one multi-agent decode-attention call. */
typedef struct {
    int32_t n_agents;                 /* >= 0; 0 is a no-op */
    int32_t n_q_heads;                /* multiple of the pools' n_kv_heads */
    int32_t layer_begin;              /* first pool layer attended */
    int32_t layer_count;              /* layers in this call (>= 0) */
    float softmax_scale;              /* 0 => 1 / sqrt(head_dim) */
    const pkv_pool* const* agent_pool;/* host [n_agents]; agents with the same pointer share a pool */
    const void* q;                    /* device [n_agents][layer_count][n_q_heads][head_dim] */
    pkv_dtype q_dtype;                /* PKV_F32 or PKV_BF16 */
    const void* sfx_k;                /* device [n_agents][layer_count][n_kv_heads][sfx_cap][head_dim] */
    const void* sfx_v;                /* same shape; both may be NULL when every sfx_len is 0 */
    pkv_dtype sfx_dtype;              /* PKV_F32 or PKV_BF16 */
    int32_t sfx_cap;                  /* suffix capacity per agent (>= max sfx_len) */
    const int32_t* sfx_len;           /* host [n_agents]: native tokens agent a attends to; may be NULL (all 0) */
    float* out;                       /* device fp32 [n_agents][layer_count][n_q_heads][head_dim] */
    int32_t kernel;                   /* pool kernel: PKV_KERNEL_DEFAULT or PKV_KERNEL_MFMA (the
                                         matrix-core kernel for any number of rows = agents * q heads
                                         per kv head: a pool with more than 64 rows, 48 with fp32
                                         queries, runs in balanced row blocks of at most that many, one
                                         workgroup each, the blocks of one (layer, kv head) on one XCD),
                                         or PKV_KERNEL_VALU (the fp32 vector kernel) */
    int32_t splits;                   /* token splits per (pool, layer, kv head); 0 = automatic */
    void* const* pool_events;         /* optional instrumentation: NULL, or two hipEvent_t recorded on
                                         the stream right before the first compressed-pool kernel
                                         (private segments, then the pool kernel) and right after the
                                         last pool-kernel launch of the call */
    const pkv_pool* const* agent_private_pool;
                                      /* optional, host [n_agents]: NULL, or per agent NULL or a second
                                         pool the agent alone (or every agent naming it) also attends:
                                         its own older tokens, quantized once when they left the
                                         native window (pool_quantize_append on that pool); it must
                                         use the same v_signs as the agent's shared pool */
} pkv_decode_args;

#define PKV_KERNEL_DEFAULT 0
#define PKV_KERNEL_VALU 1
#define PKV_KERNEL_MFMA 2

/*
 * Decode attention of every agent's query heads over its pool plus its own
 * native (uncompressed) recent tokens, for layers [layer_begin, layer_begin
 * + layer_count).  PolyKV explainer, section 2.A: agents read one shared
 * pool; section 2.B: V is dequantised by centroid lookup and inverse FWHT.
 *
 * For agent a, layer l, query head h (kv head g = h / (n_q_heads/n_kv_heads)):
 *   o = softmax(sigma * q . [K_hat; K_prv; K_sfx]) @ [V_hat; V_prv; V_sfx]
 * with K_hat = Ks * Kq and V_hat = (Vn / d) * H @ c[code] over the pool's
 * tokens, K_prv / V_prv the same over the agent's private pool when one is
 * given (CoMixKV news article, incremental quantization: recent tokens stay
 * native, older ones are quantized once and never rewritten), and the first
 * sfx_len[a] suffix tokens; no mask.  Each pool byte is
 * read once per call for all agents that share the pool (their query heads
 * are batched), V is accumulated in the rotated domain and one inverse FWHT
 * is applied per output.  fp32 accumulation.
 *
 * Query range and precision.  Any finite bf16 or fp32 query is accepted.  The
 * matrix-core pool kernel and the segment kernel take K codes as exact fp16
 * values and multiply each query row by an exact power of two 2^-e that
 * brings its largest element below 2^15 before the fp16 conversion (e > 0
 * only for rows reaching 2^15; the scores are multiplied back by 2^e), so
 * large queries neither overflow nor lose precision to an offset; bf16
 * elements more than 2^39 below their row's largest one fall into fp16's
 * subnormal range (an absolute error below 2^(e-25) each).  Scores are fp32:
 * where sigma * q . k reaches ~1e4 nats and keys are tied in their dominant
 * term, the remainder that breaks the tie is below fp32 resolution and the
 * outputs can differ from exact attention by more than 1e-3 (so does any fp32
 * computation of those scores).
 *
 * workspace: device scratch of *workspace_bytes bytes (256-byte aligned).
 * Call with workspace == NULL to have the required size written to
 * *workspace_bytes (nothing enqueued); PKV_ENOSPACE if the given size is too
 * small.  The size depends only on the call's shapes and the split plan.
 * All agents' pools, private pools included, must share n_kv_heads and
 * head_dim, hold the layers of the call, and hold the same token count in
 * each of those layers (a private pool may hold none).  q, out,
 * sfx_k and sfx_v must be 16-byte aligned (PKV_EINVAL otherwise).
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ENOSPACE, PKV_EHIP.
 */
int agent_decode_attention(const pkv_decode_args* args, void* workspace, size_t* workspace_bytes,
                           void* stream);

/*
 * agent_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same kernels and launch plan run,
 * with their partial records in a fixed device array of the library instead
 * of the workspace: pkv_noalloc_scratch_bytes() bytes (32 MiB), one copy per
 * device, held until the process ends.  Nothing is allocated by the call.
 *
 * Limit: a call whose workspace (the size agent_decode_attention reports)
 * exceeds the array returns PKV_ENOSPACE before anything is enqueued.  The
 * array keeps the previous call's contents; no kernel reads a record it has
 * not written in the same call, so nothing needs clearing.  Every call on one
 * device shares that device's array: calls that may overlap on one device
 * (different streams, or different host threads without ordering) race and
 * must be serialised by the caller.  Errors as agent_decode_attention, plus
 * PKV_EHIP if the array's device address cannot be obtained.
 */
int agent_decode_attention_noalloc(const pkv_decode_args* args, void* stream);

/* Bytes of the per-device array agent_decode_attention_noalloc uses. */
size_t pkv_noalloc_scratch_bytes(void);

/* ---- handing a pool over, and kv-head shards ---- */

/* Header of a pool image handed to another buffer, process or device: with the
 * image bytes (pool->bytes bytes from pool->base, position-independent) it
 * recreates the pool (PolyKV explainer, section 2.A: the shared context is one
 * compressed object that every agent reads).  Plain host data. */
typedef struct {
    uint32_t magic;                      /* 0x31564B50 ("PKV1") */
    int32_t abi_version;                 /* pkv_version() of the writer; the major part must match */
    pkv_pool_config cfg;
    int32_t n_tokens[PKV_MAX_LAYERS];    /* tokens stored per layer */
    uint64_t image_bytes;                /* = pool_bytes(&cfg) */
} pkv_pool_header;

/* Fill *out from a pool's descriptor.  Host only.  Errors: PKV_EINVAL. */
int pool_export_header(const pkv_pool* pool, pkv_pool_header* out);

/*
 * Describe an image whose bytes the caller has already placed at dev_buf
 * (device, 256-byte aligned, dev_bytes >= hdr->image_bytes): writes *out like
 * pool_build, with the header's token counts.  Host only, nothing enqueued.
 * Errors: PKV_EINVAL (magic, version, size or token counts inconsistent),
 * PKV_EUNSUPPORTED, PKV_ENOSPACE.
 */
int pool_import(const pkv_pool_header* hdr, void* dev_buf, size_t dev_bytes, pkv_pool* out);

/*
 * A pool holding kv heads [head_begin, head_begin + head_count) of src, laid
 * out in dev_buf (256-byte aligned, not overlapping src's buffer, dev_bytes >=
 * pool_bytes of src's config with n_kv_heads = head_count): per layer the K
 * codes, V norms, V maxima and V codes of those heads, and the K scales (all of
 * them per tensor; those heads' per token or per channel) are copied (device to
 * device, enqueued on stream); *out gets src's token counts.
 * Decoding the shard with query heads [head_begin * G, (head_begin +
 * head_count) * G) of each agent gives the outputs the whole pool gives for
 * those heads (each (layer, kv head) is decoded independently), which is how
 * a pool splits over devices.  Later appends to the shard take their K scale
 * over the shard's heads only.
 * Errors: PKV_EINVAL, PKV_ENOSPACE, PKV_EHIP (a copy could not be enqueued).
 */
int pool_shard(const pkv_pool* src, int32_t head_begin, int32_t head_count, void* dev_buf, size_t dev_bytes,
               pkv_pool* out, void* stream);

/* ---- CoMixKV controller: sensitivity and joint bit allocation ---- */

/* Arguments of one sensitivity estimate (CoMixKV news article, abstract and
 * method: per-(agent, layer) sensitivity from the recently seen queries, keys
 * and values, as a local attention-error bound, without calibration data or
 * trial quantisation). */
typedef struct {
    int32_t n_agents;                 /* >= 0; 0 is a no-op */
    int32_t layer_count;              /* >= 0 */
    int32_t n_q_heads;                /* multiple of n_kv_heads */
    int32_t n_kv_heads;               /* >= 1 */
    int32_t head_dim;                 /* 64 or 128 */
    float softmax_scale;              /* 0 => 1 / sqrt(head_dim) */
    int32_t n_recent;                 /* recent query steps per agent (>= 1) */
    const void* q;                    /* device [n_recent][n_agents][layer_count][n_q_heads][head_dim] */
    pkv_dtype q_dtype;                /* PKV_F32 or PKV_BF16 */
    const void* win_k;                /* device [n_agents][layer_count][n_kv_heads][win_cap][head_dim]:
                                         the agents' native windows (the decode call's suffix buffers) */
    const void* win_v;                /* same shape; both 16-byte aligned, may be NULL if every win_len is 0 */
    pkv_dtype win_dtype;              /* PKV_F32 or PKV_BF16 */
    int32_t win_cap;                  /* window capacity per agent */
    const int32_t* win_len;           /* host [n_agents]: tokens of agent a's window used, 0 .. win_cap */
    float* out;                       /* device fp32 [n_agents][layer_count] */
} pkv_comix_args;

/*
 * Sensitivity s[a][l] = mean over agent a's recent query rows (n_recent steps
 * x n_q_heads heads; head h uses kv head h / (n_q_heads / n_kv_heads)) of
 * sum_t p_t ||v_t||, where p = softmax_t(sigma * q . k_t) over the first
 * win_len[a] tokens of the agent's window in layer l (0 when win_len[a] = 0).
 * With a V codec of mean relative squared error D_b, the mean attention-output
 * error from quantising those values is at most sqrt(D_b) * s (triangle
 * inequality, then Jensen), which is what comix_allocate_bits weighs.
 * One workgroup per (agent, layer); deterministic (fixed summation order).
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP.
 */
int comix_sensitivity(const pkv_comix_args* args, void* stream);

/*
 * Joint V bit widths for n_items (agent, layer) items under a byte budget
 * (CoMixKV news article: 2 to 4 bits allocated over all resident agents and
 * layers under a shared budget with the real byte costs).  Host only.
 *
 * sensitivity: host [n_items], finite, >= 0 (e.g. comix_sensitivity's output);
 * cost: host [n_items][3], bytes item i's next block takes at 2, 3, 4 bits,
 * strictly increasing; error_factor: host [3], predicted error per unit of
 * sensitivity at 2, 3, 4 bits, strictly decreasing, >= 0 (sqrt of
 * pkv_lloyd_max_distortion for the bound above); bits: host [n_items] output.
 * Rule: every item starts at 2 bits; repeatedly the single upgrade b -> b + 1
 * with the largest s_i (e[b] - e[b+1]) / (cost_i[b+1] - cost_i[b]) is taken if
 * it fits the remaining budget (ties: lower index), otherwise that item stays
 * where it is; until no upgrade is left.  Returns PKV_ENOSPACE (bits
 * untouched) if 2 bits everywhere exceed the budget; PKV_EINVAL on bad input.
 */
int comix_allocate_bits(int32_t n_items, const float* sensitivity, const uint64_t* cost,
                        const double* error_factor, uint64_t budget, uint8_t* bits);

/* ---- measurement aid ---- */

/*
 * Read `bytes` bytes of device memory at src (16-byte aligned, bytes a multiple
 * of 16) with a plain streaming kernel and write the XOR of every 32-bit word,
 * folded per wavefront, to sink (device, pkv_stream_read_sink_words() words; the
 * XOR of all of them is the XOR of the buffer's words).  Not part of the decode
 * path: its time over a buffer far larger than the last-level cache is the
 * practical HBM read ceiling that the decode kernels' bandwidth is compared
 * with.  Errors: PKV_EINVAL, PKV_EHIP.
 */
int pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Words of the sink pkv_stream_read writes. */
size_t pkv_stream_read_sink_words(void);

/* ---- auxiliary queries (host only, no device work) ---- */

/* Static text for a return code. */
const char* pkv_strerror(int code);

/* ABI version: 100 * major + minor. */
int pkv_version(void);

/* sizeof of the ABI structs, for bindings to check their mirrors:
 * which = 0: pkv_pool_config, 1: pkv_pool, 2: pkv_decode_args, 3: pkv_comix_args,
 * 4: pkv_pool_header; else 0. */
size_t pkv_abi_sizeof(int32_t which);

/*
 * The library's fp32 Lloyd-Max N(0, 1) table for `bits` in {2, 3, 4}
 * (PolyKV explainer, section 2.B): centroids[2^bits] ascending and
 * thresholds[2^bits - 1] (midpoints, computed in double, then rounded).
 * Either pointer may be NULL.  Returns PKV_EUNSUPPORTED for other bits.
 */
int pkv_lloyd_max_table(int32_t bits, float* centroids, float* thresholds);

/*
 * D_b = E[(X - Q(X))^2] for X ~ N(0, 1) and the library's fp32 table at
 * `bits` in {2, 3, 4} (closed form per cell, in double); -1 for other bits.
 */
double pkv_lloyd_max_distortion(int32_t bits);

#ifdef __cplusplus
}
#endif

#endif /* POLYKV_H */
