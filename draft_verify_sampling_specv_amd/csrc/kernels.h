// Internal launchers behind the C ABI (include/specv.h).  Host code only calls these after the
// arguments have been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace specv {

constexpr int kMaxNodes = 1024;

// A per-device value computed once by `query` and cached in an atomic slot, so that concurrent
// callers may race to fill it without undefined behaviour (each computes the same value).
// Devices past the slot table are queried every time.
template <typename Query>
inline int cached_per_device(std::atomic<int> (&slots)[64], Query query) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return query(0);
    if (dev >= 64) return query(dev);
    int v = slots[dev].load(std::memory_order_relaxed);
    if (!v) {
        v = query(dev);
        slots[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Compute units of the current device (256 if the query fails).
inline int device_cu_count() {
    static std::atomic<int> cus[64];
    return cached_per_device(cus, [](int dev) {
        int n = 0;
        return (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n
                                                                                                            : 256;
    });
}

hipError_t launch_build_tree_mask(const int32_t* parent, int B, int n1, uint32_t* mask,
                                  int32_t* depth, int32_t* tree_status, hipStream_t stream);

// ------------------------------------------------------------------------------------ accept
struct AcceptArgs {
    const void* target;
    const void* draft;     // NULL iff greedy
    bool bf16;
    const int32_t* tokens;
    const int32_t* parent;
    int B, n1, V;
    float temperature;     // 0 -> greedy
    int rule;              // how siblings were drafted: 0 without replacement, 1 i.i.d., 2 fixed candidates
    uint64_t seed, offset;
    int32_t* accept_len;
    int32_t* out_tokens;
    int32_t* out_nodes;
    float* p_tok;          // may be NULL
    float* q_tok;          // may be NULL
    void* workspace;
};

size_t accept_workspace_bytes(int B, int n1, int V, bool bf16);
hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream);
// The allocation-free variant's built-in workspace: size, and its address on the current device.
constexpr size_t kAcceptScratchBytes = size_t(8) << 20;
hipError_t accept_scratch(void** ptr);

// ------------------------------------------------------------------------------------ tree expansion
constexpr int kExpandMaxK = 16;        // children per frontier node at most
constexpr int kExpandMaxCand = 1024;   // frontier rows x k per sequence at most

struct TreeExpandArgs {
    const void* logits;
    bool bf16;
    const int32_t* frontier;
    int B, F, V, k;
    float temperature;
    int keep, nmax;
    int32_t* parent;
    int32_t* tokens;
    double* score;
    int32_t* n_nodes;
    int32_t* new_frontier;
    void* workspace;
};

size_t tree_expand_workspace_bytes(int B, int F);
hipError_t launch_tree_expand(const TreeExpandArgs& a, hipStream_t stream);

// ------------------------------------------------------------------------------------ KV commit
struct KvCommitArgs {
    void* k_cache;
    void* v_cache;
    const int32_t* ctx_len;
    const int32_t* accept_len;
    const int32_t* out_nodes;
    int B, n1, Hkv, D, Lmax;
    bool bf16;
    int32_t* new_ctx_len;
};

hipError_t launch_kv_commit(const KvCommitArgs& a, hipStream_t stream);

// ------------------------------------------------------------------------------------ read probe
int read_probe_blocks();
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// ------------------------------------------------------------------------------------ attention
struct AttnArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* ctx_len;
    const uint32_t* mask;
    int B, n1, Hq, Hkv, D, Lmax;
    float scale;
    bool bf16;
    void* out;
    float* lse;            // may be NULL
    void* workspace;
};

size_t attn_workspace_bytes(int B, int n1, int Hq, int Hkv, int D, int Lmax);
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

// ------------------------------------------------------------------------------------ verify layer
struct LayerArgs {
    const void* x;             // [B n1][Hq D] bf16
    const void* w_qkv;         // [(Hq + 2 Hkv) D][Hq D]
    const void* w_o;           // [Hq D][Hq D]
    const void* w_gate_up;     // [2 inter][Hq D]
    const void* w_down;        // [Hq D][inter]
    const void* attn_norm;     // [Hq D]
    const void* mlp_norm;      // [Hq D]
    float eps, theta;
    void* k_cache;
    void* v_cache;
    const int32_t* ctx_len;
    const uint32_t* mask;
    const int32_t* depth;
    int B, n1, Hq, Hkv, D, Lmax, inter;
    void* out;
    void* workspace;
    bool packed;               // the four weight matrices in the tile order of launch_pack_weights
};

size_t layer_workspace_bytes(int B, int n1, int Hq, int Hkv, int D, int Lmax, int inter);
hipError_t launch_verify_layer(const LayerArgs& a, hipStream_t stream);
// W [N][K] bf16 (N a multiple of 32, K of 64) -> the tile order the layer's products read
hipError_t launch_pack_weights(const void* w, int N, int K, void* packed, hipStream_t stream);

// the three paths behind launch_attention
size_t attn_tree_workspace_bytes(int B, int n1, int Hq, int Hkv, int D, int Lmax);
hipError_t launch_attn_tree(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);

}  // namespace specv
