// C ABI of libspecv (declarations and full contract in include/specv.h).  Host-side argument
// validation happens here, before any launch; nothing is allocated, nothing synchronises.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "../../include/specv.h"
#include "kernels.h"

static_assert(specv::kExpandMaxK == SPECV_EXPAND_MAX_K, "expansion width limit");
static_assert(specv::kExpandMaxCand == SPECV_EXPAND_MAX_CANDIDATES, "expansion candidate limit");
static_assert(specv::kMaxNodes == SPECV_MAX_NODES, "node limit");

namespace {

thread_local char g_last_error[256] = "";

specv_status fail(specv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
specv_status fail(specv_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

specv_status ok() {
    g_last_error[0] = '\0';
    return SPECV_OK;
}

// The kernels index rows, heads and grids with 32-bit integers: a product of sizes must fit.
// (Each factor is at most 2^31 and the running product is checked before the next factor, so
// the 64-bit arithmetic itself cannot overflow.)
bool fits_i32(std::initializer_list<int64_t> factors) {
    int64_t p = 1;
    for (int64_t f : factors) {
        if (f < 0) return false;
        p *= f;
        if (p > INT32_MAX) return false;
    }
    return true;
}

bool attn_sizes_ok(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D) {
    return fits_i32({B, int64_t(K) + 1, Hq, D}) && fits_i32({B, Hkv, D});
}

bool layer_sizes_ok(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D, int32_t inter) {
    return attn_sizes_ok(B, K, Hq, Hkv, D) && fits_i32({B, int64_t(K) + 1, int64_t(Hq) + 2 * int64_t(Hkv), D}) &&
           fits_i32({B, int64_t(K) + 1, 2, inter});
}

specv_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* specv_status_string(specv_status s) {
    switch (s) {
        case SPECV_OK: return "ok";
        case SPECV_ERR_INVALID_ARG: return "invalid argument";
        case SPECV_ERR_UNSUPPORTED: return "unsupported configuration";
        case SPECV_ERR_WORKSPACE: return "workspace missing or too small";
        case SPECV_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

const char* specv_last_error(void) { return g_last_error; }

#ifdef SPECV_CHECKED
}  // extern "C"
namespace specv {
__device__ unsigned long long specv_oob_word = 0;
}  // namespace specv
extern "C" {
int64_t specv_debug_bounds(int32_t reset) {
    unsigned long long w = 0;
    if (hipDeviceSynchronize() != hipSuccess) return -2;
    if (hipMemcpyFromSymbol(&w, HIP_SYMBOL(specv::specv_oob_word), sizeof(w)) != hipSuccess) return -2;
    if (reset) {
        const unsigned long long z = 0;
        if (hipMemcpyToSymbol(HIP_SYMBOL(specv::specv_oob_word), &z, sizeof(z)) != hipSuccess) return -2;
    }
    return static_cast<int64_t>(w);
}
#else
int64_t specv_debug_bounds(int32_t) { return -1; }
#endif

specv_status specv_build_tree_mask(const int32_t* parent, int32_t B, int32_t K, uint32_t* mask,
                                   int32_t* depth, int32_t* tree_status, hipStream_t stream) {
    if (B < 0) return fail(SPECV_ERR_INVALID_ARG, "B = %d < 0", B);
    if (K < 0 || K > SPECV_MAX_NODES - 1)
        return fail(SPECV_ERR_INVALID_ARG, "K = %d outside [0, %d]", K, SPECV_MAX_NODES - 1);
    if (!fits_i32({B, int64_t(K) + 1})) return fail(SPECV_ERR_INVALID_ARG, "B * (K + 1) exceeds 2^31 - 1");
    if (B == 0) return ok();
    if (!parent || !mask || !depth || !tree_status)
        return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
    return hip_status(specv::launch_build_tree_mask(parent, B, K + 1, mask, depth, tree_status, stream),
                      "build_tree_mask");
}

size_t specv_attn_workspace_bytes(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t Lmax) {
    if (B <= 0 || K < 0 || K > SPECV_MAX_NODES - 1 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
        (D != 64 && D != 128) || Lmax <= 0 || !attn_sizes_ok(B, K, Hq, Hkv, D))
        return 0;
    return specv::attn_workspace_bytes(B, K + 1, Hq, Hkv, D, Lmax);
}

specv_status specv_tree_attn_verify(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* ctx_len, const uint32_t* mask, int32_t B,
                                    int32_t K, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax,
                                    float scale, specv_dtype dtype, void* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0) return fail(SPECV_ERR_INVALID_ARG, "B = %d < 0", B);
    if (K < 0 || K > SPECV_MAX_NODES - 1)
        return fail(SPECV_ERR_INVALID_ARG, "K = %d outside [0, %d]", K, SPECV_MAX_NODES - 1);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return fail(SPECV_ERR_INVALID_ARG, "Hq = %d, Hkv = %d: need Hq a positive multiple of Hkv", Hq, Hkv);
    if (Lmax < K + 1) return fail(SPECV_ERR_INVALID_ARG, "Lmax = %d < K + 1 = %d", Lmax, K + 1);
    if (!(std::isfinite(scale) && scale > 0.f))
        return fail(SPECV_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (dtype != SPECV_F32 && dtype != SPECV_BF16)
        return fail(SPECV_ERR_UNSUPPORTED, "dtype %d not supported", static_cast<int>(dtype));
    if (D != 64 && D != 128) return fail(SPECV_ERR_UNSUPPORTED, "head size D = %d not in {64, 128}", D);
    if (!attn_sizes_ok(B, K, Hq, Hkv, D))
        return fail(SPECV_ERR_INVALID_ARG, "B * (K + 1) * Hq * D exceeds 2^31 - 1");
    if (B == 0) return ok();
    if (!q || !k_cache || !v_cache || !ctx_len || !mask || !out)
        return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
    const size_t need = (dtype == SPECV_BF16) ? specv::attn_workspace_bytes(B, K + 1, Hq, Hkv, D, Lmax) : 0;
    if (need && (!workspace || workspace_bytes < need))
        return fail(SPECV_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    specv::AttnArgs a{q, k_cache, v_cache, ctx_len, mask, B, K + 1, Hq, Hkv, D, Lmax, scale,
                      dtype == SPECV_BF16, out, lse, workspace};
    return hip_status(specv::launch_attention(a, stream), "tree_attn_verify");
}

size_t specv_accept_workspace_bytes(int32_t B, int32_t K, int32_t V, specv_dtype logits_dtype) {
    if (B <= 0 || K < 0 || K > SPECV_MAX_NODES - 1 || V < 1 || V > SPECV_MAX_VOCAB || !fits_i32({B, int64_t(K) + 1}))
        return 0;
    return specv::accept_workspace_bytes(B, K + 1, V, logits_dtype == SPECV_BF16);
}

namespace {

// Arguments of the accept entry points, checked; on success `a` is filled (workspace unset) and
// `need` is the workspace size.  B == 0 returns SPECV_OK with a.B == 0 (nothing to launch).
specv_status accept_args(const void* target_logits, const void* draft_logits, specv_dtype logits_dtype,
                         const int32_t* tokens, const int32_t* parent, int32_t B, int32_t K, int32_t V,
                         float temperature, specv_sibling_rule rule, uint64_t seed, uint64_t offset,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes, float* p_tok, float* q_tok,
                         specv::AcceptArgs& a, size_t& need) {
    if (B < 0) return fail(SPECV_ERR_INVALID_ARG, "B = %d < 0", B);
    if (K < 0 || K > SPECV_MAX_NODES - 1)
        return fail(SPECV_ERR_INVALID_ARG, "K = %d outside [0, %d]", K, SPECV_MAX_NODES - 1);
    if (V < 1 || V > SPECV_MAX_VOCAB)
        return fail(SPECV_ERR_INVALID_ARG, "V = %d outside [1, %d]", V, SPECV_MAX_VOCAB);
    if (!std::isfinite(temperature) || temperature < 0.f)
        return fail(SPECV_ERR_INVALID_ARG, "temperature must be finite and >= 0");
    if (rule != SPECV_SIBLINGS_WITHOUT_REPLACEMENT && rule != SPECV_SIBLINGS_IID &&
        rule != SPECV_SIBLINGS_DETERMINISTIC)
        return fail(SPECV_ERR_INVALID_ARG, "sibling rule %d not in {0, 1, 2}", static_cast<int>(rule));
    if (logits_dtype != SPECV_F32 && logits_dtype != SPECV_BF16)
        return fail(SPECV_ERR_UNSUPPORTED, "dtype %d not supported", static_cast<int>(logits_dtype));
    if (!fits_i32({B, int64_t(K) + 1})) return fail(SPECV_ERR_INVALID_ARG, "B * (K + 1) exceeds 2^31 - 1");
    a = specv::AcceptArgs{};
    need = 0;
    if (B == 0) return ok();
    if (!target_logits || !tokens || !parent || !accept_len || !out_tokens || !out_nodes)
        return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
    const bool need_draft = temperature > 0.f && rule != SPECV_SIBLINGS_DETERMINISTIC;
    if (need_draft && !draft_logits)
        return fail(SPECV_ERR_INVALID_ARG,
                    "draft_logits may be NULL only at temperature 0 or for deterministic siblings");
    need = specv::accept_workspace_bytes(B, K + 1, V, logits_dtype == SPECV_BF16);
    a = specv::AcceptArgs{target_logits, need_draft ? draft_logits : nullptr,
                          logits_dtype == SPECV_BF16, tokens, parent, B, K + 1, V, temperature,
                          static_cast<int>(rule), seed, offset, accept_len, out_tokens, out_nodes, p_tok, q_tok,
                          nullptr};
    return SPECV_OK;
}

}  // namespace

specv_status specv_accept_resample_rule(const void* target_logits, const void* draft_logits,
                                        specv_dtype logits_dtype, const int32_t* tokens,
                                        const int32_t* parent, int32_t B, int32_t K, int32_t V,
                                        float temperature, specv_sibling_rule rule, uint64_t seed,
                                        uint64_t offset, int32_t* accept_len, int32_t* out_tokens,
                                        int32_t* out_nodes, float* p_tok, float* q_tok, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    specv::AcceptArgs a;
    size_t need = 0;
    const specv_status st = accept_args(target_logits, draft_logits, logits_dtype, tokens, parent, B, K, V,
                                        temperature, rule, seed, offset, accept_len, out_tokens, out_nodes, p_tok,
                                        q_tok, a, need);
    if (st != SPECV_OK || a.B == 0) return st;
    if (!workspace || workspace_bytes < need)
        return fail(SPECV_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    a.workspace = workspace;
    return hip_status(specv::launch_accept(a, stream), "accept_resample");
}

specv_status specv_accept_resample_rule_noalloc(const void* target_logits, const void* draft_logits,
                                                specv_dtype logits_dtype, const int32_t* tokens,
                                                const int32_t* parent, int32_t B, int32_t K, int32_t V,
                                                float temperature, specv_sibling_rule rule, uint64_t seed,
                                                uint64_t offset, int32_t* accept_len, int32_t* out_tokens,
                                                int32_t* out_nodes, float* p_tok, float* q_tok,
                                                hipStream_t stream) {
    specv::AcceptArgs a;
    size_t need = 0;
    const specv_status st = accept_args(target_logits, draft_logits, logits_dtype, tokens, parent, B, K, V,
                                        temperature, rule, seed, offset, accept_len, out_tokens, out_nodes, p_tok,
                                        q_tok, a, need);
    if (st != SPECV_OK || a.B == 0) return st;
    if (need > specv::kAcceptScratchBytes)
        return fail(SPECV_ERR_WORKSPACE, "this call needs %zu bytes of workspace; the built-in one holds %zu",
                    need, specv::kAcceptScratchBytes);
    void* ws = nullptr;
    const hipError_t e = specv::accept_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "accept_resample_noalloc (workspace address)");
    a.workspace = ws;
    return hip_status(specv::launch_accept(a, stream), "accept_resample_noalloc");
}

specv_status specv_accept_resample(const void* target_logits, const void* draft_logits,
                                   specv_dtype logits_dtype, const int32_t* tokens,
                                   const int32_t* parent, int32_t B, int32_t K, int32_t V,
                                   float temperature, uint64_t seed, uint64_t offset,
                                   int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes,
                                   float* p_tok, float* q_tok, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    return specv_accept_resample_rule(target_logits, draft_logits, logits_dtype, tokens, parent, B, K, V,
                                      temperature, SPECV_SIBLINGS_WITHOUT_REPLACEMENT, seed, offset,
                                      accept_len, out_tokens, out_nodes, p_tok, q_tok, workspace,
                                      workspace_bytes, stream);
}

size_t specv_tree_expand_workspace_bytes(int32_t B, int32_t F) {
    if (B <= 0 || F <= 0 || !fits_i32({B, F})) return 0;
    return specv::tree_expand_workspace_bytes(B, F);
}

specv_status specv_tree_expand(const void* draft_logits, specv_dtype dtype, const int32_t* frontier,
                               int32_t B, int32_t F, int32_t V, int32_t k, float temperature,
                               int32_t keep, int32_t nmax, int32_t* parent, int32_t* tokens,
                               double* score, int32_t* n_nodes, int32_t* new_frontier, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    if (B < 0) return fail(SPECV_ERR_INVALID_ARG, "B = %d < 0", B);
    if (F < 1) return fail(SPECV_ERR_INVALID_ARG, "F = %d < 1", F);
    if (V < 1 || V > SPECV_MAX_VOCAB)
        return fail(SPECV_ERR_INVALID_ARG, "V = %d outside [1, %d]", V, SPECV_MAX_VOCAB);
    if (k < 1 || k > SPECV_EXPAND_MAX_K)
        return fail(SPECV_ERR_INVALID_ARG, "k = %d outside [1, %d]", k, SPECV_EXPAND_MAX_K);
    if (static_cast<int64_t>(F) * k > SPECV_EXPAND_MAX_CANDIDATES)
        return fail(SPECV_ERR_INVALID_ARG, "F * k = %lld > %d", static_cast<long long>(F) * k,
                    SPECV_EXPAND_MAX_CANDIDATES);
    if (!std::isfinite(temperature) || temperature <= 0.f)
        return fail(SPECV_ERR_INVALID_ARG, "temperature must be finite and > 0");
    if (keep < 1 || keep > SPECV_MAX_NODES)
        return fail(SPECV_ERR_INVALID_ARG, "keep = %d outside [1, %d]", keep, SPECV_MAX_NODES);
    if (nmax < 1 || nmax > SPECV_MAX_NODES)
        return fail(SPECV_ERR_INVALID_ARG, "nmax = %d outside [1, %d]", nmax, SPECV_MAX_NODES);
    if (dtype != SPECV_F32 && dtype != SPECV_BF16)
        return fail(SPECV_ERR_UNSUPPORTED, "dtype %d not supported", static_cast<int>(dtype));
    if (!fits_i32({B, F})) return fail(SPECV_ERR_INVALID_ARG, "B * F exceeds 2^31 - 1");
    if (B == 0) return ok();
    if (!draft_logits || !frontier || !parent || !tokens || !score || !n_nodes || !new_frontier)
        return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
    const size_t need = specv::tree_expand_workspace_bytes(B, F);
    if (!workspace || workspace_bytes < need)
        return fail(SPECV_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    specv::TreeExpandArgs a{draft_logits, dtype == SPECV_BF16, frontier, B, F, V, k, temperature, keep, nmax,
                            parent, tokens, score, n_nodes, new_frontier, workspace};
    return hip_status(specv::launch_tree_expand(a, stream), "tree_expand");
}

specv_status specv_kv_commit(void* k_cache, void* v_cache, const int32_t* ctx_len,
                             const int32_t* accept_len, const int32_t* out_nodes, int32_t B,
                             int32_t K, int32_t Hkv, int32_t D, int32_t Lmax, specv_dtype dtype,
                             int32_t* new_ctx_len, hipStream_t stream) {
    if (B < 0) return fail(SPECV_ERR_INVALID_ARG, "B = %d < 0", B);
    if (K < 0 || K > SPECV_MAX_NODES - 1)
        return fail(SPECV_ERR_INVALID_ARG, "K = %d outside [0, %d]", K, SPECV_MAX_NODES - 1);
    if (Hkv <= 0) return fail(SPECV_ERR_INVALID_ARG, "Hkv = %d <= 0", Hkv);
    if (Lmax < K + 1) return fail(SPECV_ERR_INVALID_ARG, "Lmax = %d < K + 1 = %d", Lmax, K + 1);
    if (dtype != SPECV_F32 && dtype != SPECV_BF16)
        return fail(SPECV_ERR_UNSUPPORTED, "dtype %d not supported", static_cast<int>(dtype));
    if (D != 64 && D != 128) return fail(SPECV_ERR_UNSUPPORTED, "head size D = %d not in {64, 128}", D);
    if (!fits_i32({B, int64_t(K) + 1, 2, Hkv})) return fail(SPECV_ERR_INVALID_ARG, "B * (K + 1) * 2 * Hkv exceeds 2^31 - 1");
    if (B == 0) return ok();
    if (!k_cache || !v_cache || !ctx_len || !accept_len || !out_nodes || !new_ctx_len)
        return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
    if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15)
        return fail(SPECV_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
    specv::KvCommitArgs a{k_cache, v_cache, ctx_len, accept_len, out_nodes, B, K + 1, Hkv, D, Lmax,
                          dtype == SPECV_BF16, new_ctx_len};
    return hip_status(specv::launch_kv_commit(a, stream), "kv_commit");
}

int32_t specv_read_probe_sink_words(void) { return specv::read_probe_blocks(); }

specv_status specv_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                              hipStream_t stream) {
    if (bytes == 0) return ok();
    if (!buf || !sink) return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
    if ((reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15))
        return fail(SPECV_ERR_INVALID_ARG, "buf and bytes must be multiples of 16");
    if (sink_words < static_cast<size_t>(specv::read_probe_blocks()))
        return fail(SPECV_ERR_INVALID_ARG, "sink holds %zu words, needs %d", sink_words, specv::read_probe_blocks());
    return hip_status(specv::launch_read_probe(buf, bytes, sink, stream), "read_probe");
}

size_t specv_verify_layer_workspace_bytes(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                                          int32_t Lmax, int32_t inter) {
    if (B <= 0 || K < 0 || K > SPECV_MAX_NODES - 1 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
        (D != 64 && D != 128) || Lmax < K + 1 || inter <= 0 || inter % 64 != 0 ||
        !layer_sizes_ok(B, K, Hq, Hkv, D, inter))
        return 0;
    return specv::layer_workspace_bytes(B, K + 1, Hq, Hkv, D, Lmax, inter);
}

}  // extern "C"

namespace {

specv_status verify_layer_call(const void* x, const void* w_qkv, const void* w_o, const void* w_gate_up,
                               const void* w_down, const void* attn_norm, const void* mlp_norm,
                               float rms_eps, float rope_theta, void* k_cache, void* v_cache,
                               const int32_t* ctx_len, const uint32_t* mask, const int32_t* depth,
                               int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax,
                               int32_t inter, void* out, void* workspace, size_t workspace_bytes,
                               bool packed, hipStream_t stream) {
    if (B < 0) return fail(SPECV_ERR_INVALID_ARG, "B = %d < 0", B);
    if (K < 0 || K > SPECV_MAX_NODES - 1)
        return fail(SPECV_ERR_INVALID_ARG, "K = %d outside [0, %d]", K, SPECV_MAX_NODES - 1);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return fail(SPECV_ERR_INVALID_ARG, "Hq = %d, Hkv = %d: need Hq a positive multiple of Hkv", Hq, Hkv);
    if (Lmax < K + 1) return fail(SPECV_ERR_INVALID_ARG, "Lmax = %d < K + 1 = %d", Lmax, K + 1);
    if (inter <= 0 || inter % 64 != 0)
        return fail(SPECV_ERR_INVALID_ARG, "inter = %d is not a positive multiple of 64", inter);
    if (!(std::isfinite(rms_eps) && rms_eps > 0.f)) return fail(SPECV_ERR_INVALID_ARG, "rms_eps must be > 0");
    if (!(std::isfinite(rope_theta) && rope_theta > 1.f))
        return fail(SPECV_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
    if (D != 64 && D != 128) return fail(SPECV_ERR_UNSUPPORTED, "head size D = %d not in {64, 128}", D);
    if (!layer_sizes_ok(B, K, Hq, Hkv, D, inter))
        return fail(SPECV_ERR_INVALID_ARG, "row, head or MLP sizes exceed 2^31 - 1 elements");
    if (B == 0) return ok();
    const void* ptrs[] = {x, w_qkv, w_o, w_gate_up, w_down, attn_norm, mlp_norm, k_cache, v_cache, out};
    for (const void* p : ptrs) {
        if (!p) return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
        if (reinterpret_cast<uintptr_t>(p) & 15)
            return fail(SPECV_ERR_INVALID_ARG, "weights, activations and caches must be 16-byte aligned");
    }
    if (!ctx_len || !mask || !depth) return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
    const size_t need = specv::layer_workspace_bytes(B, K + 1, Hq, Hkv, D, Lmax, inter);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255))
        return fail(SPECV_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need,
                    workspace_bytes);
    specv::LayerArgs a{x, w_qkv, w_o, w_gate_up, w_down, attn_norm, mlp_norm, rms_eps, rope_theta,
                       k_cache, v_cache, ctx_len, mask, depth, B, K + 1, Hq, Hkv, D, Lmax, inter, out,
                       workspace, packed};
    return hip_status(specv::launch_verify_layer(a, stream), "verify_layer");
}

}  // namespace

extern "C" {

specv_status specv_verify_layer(const void* x, const void* w_qkv, const void* w_o, const void* w_gate_up,
                                const void* w_down, const void* attn_norm, const void* mlp_norm,
                                float rms_eps, float rope_theta, void* k_cache, void* v_cache,
                                const int32_t* ctx_len, const uint32_t* mask, const int32_t* depth,
                                int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax,
                                int32_t inter, void* out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    return verify_layer_call(x, w_qkv, w_o, w_gate_up, w_down, attn_norm, mlp_norm, rms_eps, rope_theta, k_cache,
                             v_cache, ctx_len, mask, depth, B, K, Hq, Hkv, D, Lmax, inter, out, workspace,
                             workspace_bytes, false, stream);
}

specv_status specv_verify_layer_packed(const void* x, const void* w_qkv, const void* w_o, const void* w_gate_up,
                                       const void* w_down, const void* attn_norm, const void* mlp_norm,
                                       float rms_eps, float rope_theta, void* k_cache, void* v_cache,
                                       const int32_t* ctx_len, const uint32_t* mask, const int32_t* depth,
                                       int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax,
                                       int32_t inter, void* out, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    return verify_layer_call(x, w_qkv, w_o, w_gate_up, w_down, attn_norm, mlp_norm, rms_eps, rope_theta, k_cache,
                             v_cache, ctx_len, mask, depth, B, K, Hq, Hkv, D, Lmax, inter, out, workspace,
                             workspace_bytes, true, stream);
}

specv_status specv_pack_weights(const void* w, int32_t N, int32_t K, void* packed, hipStream_t stream) {
    if (N <= 0 || N % 32 != 0) return fail(SPECV_ERR_INVALID_ARG, "N = %d is not a positive multiple of 32", N);
    if (K <= 0 || K % 64 != 0) return fail(SPECV_ERR_INVALID_ARG, "K = %d is not a positive multiple of 64", K);
    if (!w || !packed) return fail(SPECV_ERR_INVALID_ARG, "NULL pointer argument");
    if ((reinterpret_cast<uintptr_t>(w) & 15) || (reinterpret_cast<uintptr_t>(packed) & 15))
        return fail(SPECV_ERR_INVALID_ARG, "w and packed must be 16-byte aligned");
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(w), b0 = reinterpret_cast<uintptr_t>(packed);
    const uintptr_t bytes = static_cast<uintptr_t>(N) * static_cast<uintptr_t>(K) * 2u;
    if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(SPECV_ERR_INVALID_ARG, "w and packed overlap");
    return hip_status(specv::launch_pack_weights(w, N, K, packed, stream), "pack_weights");
}

}  // extern "C"
