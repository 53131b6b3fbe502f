// One level of draft-tree expansion: each frontier node proposes the k tokens of highest draft
// probability, and of all candidates of a sequence the `keep` with the highest cumulative draft
// log-probability are appended to the tree.
//
// [SD-EAGLE] "EAGLE: tree drafting and feature reuse": the draft outputs K candidates per depth
// (exercise 4: the top 3 branches at every depth); EAGLE-2 grows the tree wide where the draft is
// unsure and narrow where it is confident.  [PTD] Method 2, "Progressive Expansion & Pruning":
// each step drafts children for all current leaves in one pass; width control caps the children
// per parent.
//
//   expand_topk_kernel   one 16-wave workgroup per frontier row: one coalesced pass over the row
//                        (batches of four 16-byte loads per thread, the next batch in flight while
//                        one is processed) keeps a per-thread top-k in registers -- a batch is
//                        examined only if its max would enter -- and the online log-sum-exp of
//                        z / T (scaled reference, one fma per term, one rescale per vector); k rounds of a
//                        wave-wide argmax over the lanes' list heads merge each wave, and one wave
//                        merges the waves' lists through LDS.  HBM-bound: each row is read once.
//   expand_select_kernel one workgroup per sequence: the rank of every candidate (score, then
//                        frontier row, then rank within the row) by counting, the `keep` best
//                        survive (fewer at the node capacity) and are appended in frontier / rank
//                        order.
//
// Ties: equal logits go to the lower token id; equal scores to the earlier row, then the better
// rank.  Scores are fp64 (the row's log-sum-exp is combined in fp64 from fp32 per-thread sums).

#include <cfloat>
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace specv {
namespace {

constexpr int kTopThreads = 1024;           // 16 waves per row: enough loads in flight
constexpr int kTopWaves = kTopThreads / kWave;
constexpr int kBatch = 4;                   // 16-byte vectors per thread loaded together
constexpr int kSelThreads = 512;
constexpr double kLn2d = 0.6931471805599453;

struct RowTop {              // per-row result in the workspace
    int32_t tok[kExpandMaxK];
    float z[kExpandMaxK];
    double lse;              // log sum exp(z / T) over the row
    int32_t count;           // candidates of the row (0: no row)
    int32_t pad;
};

// The elements of one 16-byte vector as fp32 (bf16: its bits in the high half of a word; exact).
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& r, float* out);
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& r, float* out) {
    out[0] = __uint_as_float(r.x); out[1] = __uint_as_float(r.y);
    out[2] = __uint_as_float(r.z); out[3] = __uint_as_float(r.w);
}
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& r, float* out) {
    out[0] = bf16_lo(r.x); out[1] = bf16_hi(r.x); out[2] = bf16_lo(r.y); out[3] = bf16_hi(r.y);
    out[4] = bf16_lo(r.z); out[5] = bf16_hi(r.z); out[6] = bf16_lo(r.w); out[7] = bf16_hi(r.w);
}

// (value, index) order: larger value first, then lower index
__device__ __forceinline__ bool better(float v, int i, float v2, int i2) {
    return v > v2 || (v == v2 && i < i2);
}

// One DPP step of the wave maximum: v against the lane that the DPP control kCtrl selects.
template <int kCtrl>
__device__ __forceinline__ float dpp_max_step(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false)));
}

// Maximum over the wave through DPP: rows of 16 lanes reduce with quad permutations and row
// rotations (every lane of a row ends with the row's maximum), then the four row maxima are read
// as scalars.  Unlike a shuffle through the LDS crossbar, no step waits on a memory counter.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = dpp_max_step<0xB1>(v);     // quad_perm 1,0,3,2
    v = dpp_max_step<0x4E>(v);     // quad_perm 2,3,0,1
    v = dpp_max_step<0x124>(v);    // row_ror 4
    v = dpp_max_step<0x128>(v);    // row_ror 8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The kk-th largest of v over the wave (counting repeats): kk rounds, each removing the largest
// (one lane at a time).
__device__ __forceinline__ float wave_kth_largest(float v, int kk, int lane) {
    float cur = -INFINITY;
    for (int r = 0; r < kk; ++r) {
        cur = wave_max_dpp(v);
        const uint64_t at = __ballot(v == cur);
        if (at && lane == __ffsll(static_cast<unsigned long long>(at)) - 1) v = -INFINITY;
    }
    return cur;
}

// K: capacity of the per-thread lists (k <= K); a list keeps its thread's K best entered elements
template <typename T, int K>
__global__ void __launch_bounds__(kTopThreads)
expand_topk_kernel(const T* __restrict__ logits, const int32_t* __restrict__ frontier,
                   const int32_t* __restrict__ n_nodes, int F, int V, int k, int nmax, float kexp2,
                   double invT, RowTop* __restrict__ rows) {
    constexpr int kVec = Elem<T>::kVec;
    __shared__ float lv[kTopWaves][K];
    __shared__ int li[kTopWaves][K];
    __shared__ float wm[kTopWaves], ws[kTopWaves];
    const int row = blockIdx.x, b = row / F;
    const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
    RowTop* out = rows + row;
    const T* z = logits + static_cast<int64_t>(row) * V;
    const int kk = min(k, V);
    constexpr int kStep = kTopThreads * kVec;
    constexpr int kBatchElems = kBatch * kStep;
    const bool vec = (V % kVec) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0;
    // batches whose vectors all lie inside the row: loaded unconditionally, no bounds selects
    const int nfull = vec ? V / kBatchElems : 0;
    uint4 r[kBatch];
    auto load_full = [&](int b0) {
#pragma unroll
        for (int q = 0; q < kBatch; ++q) r[q] = *reinterpret_cast<const uint4*>(z + b0 + q * kStep + t * kVec);
    };
    // the first full batch is requested before the frontier entry and the node count, so that
    // their round trip overlaps it (a row that is no node has then loaded it for nothing; it lies
    // inside the logits either way).  Those two are vector loads issued after it: read as scalar
    // loads they would be waited for before anything else is issued.
    if (nfull > 0) load_full(0);
    const int u = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(frontier + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    const int n = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(n_nodes + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (!(u >= 0 && u < min(n, nmax))) { // (workgroup-uniform) not a node: no row
        if (t == 0) out->count = 0;
        return;
    }

    // per-thread list of the K best entered elements, sorted (value desc, index asc); this
    // thread's elements come in increasing index order, so a strictly larger value is needed to
    // displace the K-th
    float tv[K];
    int ti[K];
#pragma unroll
    for (int j = 0; j < K; ++j) { tv[j] = -INFINITY; ti[j] = INT_MAX; }
    float wthr = -INFINITY;              // the wave-wide entry bound (see below)
    int held = 0;
    // online log-sum-exp in the scaled domain: R the largest x kexp2 so far (never below
    // -FLT_MAX), s the sum of exp2(x kexp2 - R), each argument one fma
    float R = -FLT_MAX, s = 0.f;
    auto insert = [&](float x, int xi) {
        ++held;
        float cv = x;
        int ci = xi;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const bool go = better(cv, ci, tv[j], ti[j]);
            const float ov = tv[j];
            const int oi = ti[j];
            tv[j] = go ? cv : ov;
            ti[j] = go ? ci : oi;
            cv = go ? ov : cv;
            ci = go ? oi : ci;
        }
    };
    // one batch of kBatch vectors per thread: the online log-sum-exp, the wave-wide entry bound,
    // and the insertions.  tail: the batch may reach past V (its elements there are -inf).
    auto process = [&](int b0, float (&x)[kBatch][kVec], bool tail) {
        float vm[kBatch];
        float bmax = -INFINITY;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            vm[q] = x[q][0];
#pragma unroll
            for (int e = 1; e < kVec; ++e) vm[q] = fmaxf(vm[q], x[q][e]);
            // online log-sum-exp, one rescale per vector
            const float Rn = fmaxf(R, vm[q] * kexp2);
            float add = 0.f;
#pragma unroll
            for (int e = 0; e < kVec; ++e) add += __builtin_amdgcn_exp2f(__builtin_fmaf(x[q][e], kexp2, -Rn));
            s = __builtin_fmaf(s, __builtin_amdgcn_exp2f(R - Rn), add);
            R = Rn;
            bmax = fmaxf(bmax, vm[q]);
        }
        // wave-wide entry bound: the kk-th largest of the lanes' batch maxima -- kk elements at
        // or above it exist, so anything below it cannot be in the wave's top-k (equal values may
        // still be, on index); it only grows.  A vector is scanned only if its maximum reaches it.
        wthr = fmaxf(wthr, wave_kth_largest(bmax, kk, lane));
        if (bmax >= wthr) {
            const float thr = tv[K - 1];          // -inf while the list is not full
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                if (vm[q] >= wthr) {
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        const int i = b0 + q * kStep + t * kVec + e;
                        if ((!tail || i < V) && x[q][e] >= wthr && (held < K || x[q][e] > thr)) insert(x[q][e], i);
                    }
                }
        }
    };
    for (int bi = 0; bi < nfull; ++bi) {
        float x[kBatch][kVec];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) unpack16<T>(r[q], x[q]);
        // the next batch is in flight while this one is processed
        if (bi + 1 < nfull) load_full((bi + 1) * kBatchElems);
        process(bi * kBatchElems, x, false);
    }
    // the rest of the row (and every batch of a row without 16-byte vectors): bounds-checked
    for (int b0 = nfull * kBatchElems; b0 < V; b0 += kBatchElems) {
        float x[kBatch][kVec];
        if (vec) {
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int base = b0 + q * kStep + t * kVec;
                r[q] = make_uint4(0, 0, 0, 0);
                if (base < V) r[q] = *reinterpret_cast<const uint4*>(z + base);
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int base = b0 + q * kStep + t * kVec;
                float y[kVec];
                unpack16<T>(r[q], y);
#pragma unroll
                for (int e = 0; e < kVec; ++e) x[q][e] = base < V ? y[e] : -INFINITY;
            }
        } else {
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    const int i = b0 + q * kStep + t * kVec + e;
                    x[q][e] = i < V ? Elem<T>::load(z, i) : -INFINITY;
                }
        }
        process(b0, x, true);
    }

    // per wave: kk rounds, each taking the best head of the lanes' sorted lists (the winning lane
    // shifts its list up by one)
    wave_max_sum(R, s, 1.0f);            // (references already scaled)
    if (lane == 0) { wm[w] = R; ws[w] = s; }
    for (int r = 0; r < kk; ++r) {
        float bv = tv[0];
        int bi = ti[0], bl = (ti[0] == INT_MAX) ? -1 : lane;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float v2 = __shfl_xor(bv, o);
            const int i2 = __shfl_xor(bi, o), l2 = __shfl_xor(bl, o);
            if (l2 >= 0 && (bl < 0 || better(v2, i2, bv, bi))) { bv = v2; bi = i2; bl = l2; }
        }
        if (lane == bl) {
#pragma unroll
            for (int j = 0; j + 1 < K; ++j) { tv[j] = tv[j + 1]; ti[j] = ti[j + 1]; }
            tv[K - 1] = -INFINITY;
            ti[K - 1] = INT_MAX;
        }
        if (lane == 0) {
            lv[w][r] = bv;
            li[w][r] = bl >= 0 ? bi : INT_MAX;
        }
    }
    __syncthreads();
    if (w == 0) {
        // across waves: up to kTopWaves x kk candidates, kTopWaves * kExpandMaxK / 64 per lane
        constexpr int kPer = (kTopWaves * K + kWave - 1) / kWave;
        float cv[kPer];
        int ci[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = q * kWave + lane, ww = e / K, rr = e % K;
            const bool ok = ww < kTopWaves && rr < kk;
            cv[q] = ok ? lv[min(ww, kTopWaves - 1)][rr] : -INFINITY;
            ci[q] = ok ? li[min(ww, kTopWaves - 1)][rr] : INT_MAX;
        }
        for (int r = 0; r < kk; ++r) {
            float bv = -INFINITY;
            int bi = INT_MAX, bq = -1;
#pragma unroll
            for (int q = 0; q < kPer; ++q)
                if (ci[q] != INT_MAX && (bq < 0 || better(cv[q], ci[q], bv, bi))) { bv = cv[q]; bi = ci[q]; bq = q; }
            int bl = bq >= 0 ? lane : -1;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float v2 = __shfl_xor(bv, o);
                const int i2 = __shfl_xor(bi, o), l2 = __shfl_xor(bl, o);
                if (l2 >= 0 && (bl < 0 || better(v2, i2, bv, bi))) { bv = v2; bi = i2; bl = l2; }
            }
            if (lane == bl) {
#pragma unroll
                for (int q = 0; q < kPer; ++q)
                    if (q == bq) ci[q] = INT_MAX;
            }
            if (lane == 0) {
                out->tok[r] = bi;
                out->z[r] = bv;
            }
        }
        if (lane == 0) {
            float M = -INFINITY;
            for (int q = 0; q < kTopWaves; ++q) M = fmaxf(M, wm[q]);
            double S = 0.0;
            for (int q = 0; q < kTopWaves; ++q) S += static_cast<double>(ws[q]) * exp2(static_cast<double>(wm[q]) - M);
            out->lse = static_cast<double>(M) * kLn2d + log(S);
            out->count = kk;
        }
    }
}

__global__ void __launch_bounds__(kSelThreads)
expand_select_kernel(const RowTop* __restrict__ rows, const int32_t* __restrict__ frontier, int F, int k,
                     int keep, int nmax, double invT, int32_t* __restrict__ parent, int32_t* __restrict__ tokens,
                     double* __restrict__ score, int32_t* __restrict__ n_nodes, int32_t* __restrict__ new_frontier) {
    __shared__ double cs[kExpandMaxCand];
    __shared__ int wcnt[kSelThreads / kWave];
    __shared__ int s_total;
    const int b = blockIdx.x, t = threadIdx.x, lane = t % kWave, w = t / kWave;
    const int C = F * k;
    const int n = n_nodes[b];
    const RowTop* rb = rows + static_cast<int64_t>(b) * F;
    const int64_t tb = static_cast<int64_t>(b) * nmax;
    // candidate c = f * k + j; invalid candidates (no row, j >= count) get -inf and are never kept
    for (int c = t; c < C; c += kSelThreads) {
        const int f = c / k, j = c % k;
        const RowTop& r = rb[f];
        double sc = -INFINITY;
        if (j < r.count)
            sc = score[tb + SPECV_CHK(frontier[b * F + f], nmax, kSiteExpandFrontier)] + (static_cast<double>(r.z[j]) * invT - r.lse);
        cs[c] = sc;
    }
    if (t == 0) s_total = 0;
    __syncthreads();
    int valid = 0;
    for (int c = t; c < C; c += kSelThreads) valid += (cs[c] != -INFINITY);
    atomicAdd(&s_total, valid);
    __syncthreads();
    const int M = max(0, min(min(keep, s_total), nmax - n));
    // kept: rank < M, the rank counting every candidate ahead in (score desc, index asc)
    int done = 0;
    for (int c0 = 0; c0 < C; c0 += kSelThreads) {
        const int c = c0 + t;
        bool kept = false;
        if (c < C && cs[c] != -INFINITY) {
            const double sc = cs[c];
            int rank = 0;
            for (int d = 0; d < C; ++d) {
                const double o = cs[d];
                rank += (o > sc || (o == sc && d < c)) ? 1 : 0;
            }
            kept = rank < M;
        }
        // position among the kept, in index order (= frontier row, then rank in the row)
        const uint64_t bal = __ballot(kept);
        if (lane == 0) wcnt[w] = __popcll(bal);
        __syncthreads();
        int before = done;
        int all = 0;
        for (int q = 0; q < kSelThreads / kWave; ++q) {
            if (q < w) before += wcnt[q];
            all += wcnt[q];
        }
        if (kept) {
            const int pos = before + __popcll(bal & ((1ull << lane) - 1ull));
            const int f = c / k, j = c % k;
            const int node = SPECV_CHK(n + pos, nmax, kSiteExpandNode);
            parent[tb + node] = frontier[b * F + f];
            tokens[tb + node] = rb[f].tok[j];
            score[tb + node] = cs[c];
            new_frontier[static_cast<int64_t>(b) * keep + SPECV_CHK(pos, keep, kSiteExpandPos)] = node;
        }
        done += all;
        __syncthreads();
    }
    for (int i = M + t; i < keep; i += kSelThreads) new_frontier[static_cast<int64_t>(b) * keep + i] = -1;
    if (t == 0) n_nodes[b] = n + M;
}

template <typename T, int K>
void launch_topk(const TreeExpandArgs& a, const T* z, float kexp2, double invT, RowTop* rows, hipStream_t stream) {
    hipLaunchKernelGGL((expand_topk_kernel<T, K>), dim3(a.B * a.F), dim3(kTopThreads), 0, stream, z, a.frontier,
                       a.n_nodes, a.F, a.V, a.k, a.nmax, kexp2, invT, rows);
}

}  // namespace

size_t tree_expand_workspace_bytes(int B, int F) { return sizeof(RowTop) * static_cast<size_t>(B) * F; }

hipError_t launch_tree_expand(const TreeExpandArgs& a, hipStream_t stream) {
    RowTop* rows = static_cast<RowTop*>(a.workspace);
    const double invT = 1.0 / static_cast<double>(a.temperature);
    const float kexp2 = static_cast<float>(1.4426950408889634 * invT);
    if (a.bf16) {
        const uint16_t* z = static_cast<const uint16_t*>(a.logits);
        if (a.k <= 4) launch_topk<uint16_t, 4>(a, z, kexp2, invT, rows, stream);
        else if (a.k <= 8) launch_topk<uint16_t, 8>(a, z, kexp2, invT, rows, stream);
        else launch_topk<uint16_t, 16>(a, z, kexp2, invT, rows, stream);
    } else {
        const float* z = static_cast<const float*>(a.logits);
        if (a.k <= 4) launch_topk<float, 4>(a, z, kexp2, invT, rows, stream);
        else if (a.k <= 8) launch_topk<float, 8>(a, z, kexp2, invT, rows, stream);
        else launch_topk<float, 16>(a, z, kexp2, invT, rows, stream);
    }
    hipLaunchKernelGGL(expand_select_kernel, dim3(a.B), dim3(kSelThreads), 0, stream, rows, a.frontier, a.F, a.k,
                       a.keep, a.nmax, invT, a.parent, a.tokens, a.score, a.n_nodes, a.new_frontier);
    return hipGetLastError();
}

}  // namespace specv
