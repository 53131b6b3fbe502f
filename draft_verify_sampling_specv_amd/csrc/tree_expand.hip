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
//   expand_topk_kernel   one workgroup per frontier row: one coalesced pass over the row keeps a
//                        per-thread top-k (registers) and the online (max, sum of exp) of z / T;
//                        the workgroup merges the per-thread lists in LDS (k rounds of a
//                        wave-wide argmax over the lists' heads).  HBM-bound: each row is read once.
//   expand_select_kernel one workgroup per sequence: the rank of every candidate (score, then
//                        frontier row, then rank within the row) by counting, the `keep` best
//                        survive (fewer at the node capacity) and are appended in frontier / rank
//                        order.
//
// Ties: equal logits go to the lower token id; equal scores to the earlier row, then the better
// rank.  Scores are fp64 (the row's log-sum-exp is combined in fp64 from fp32 per-thread sums).

#include <cmath>

#include "common.h"
#include "kernels.h"

namespace specv {
namespace {

constexpr int kTopThreads = 256;
constexpr int kTopWaves = kTopThreads / kWave;
constexpr int kSelThreads = 512;

struct RowTop {              // per-row result in the workspace
    int32_t tok[kExpandMaxK];
    float z[kExpandMaxK];
    double lse;              // log sum exp(z / T) over the row
    int32_t count;           // candidates of the row (0: no row)
    int32_t pad;
};

// (value, index) order: larger value first, then lower index
__device__ __forceinline__ bool better(float v, int i, float v2, int i2) {
    return v > v2 || (v == v2 && i < i2);
}

template <typename T>
__global__ void __launch_bounds__(kTopThreads)
expand_topk_kernel(const T* __restrict__ logits, const int32_t* __restrict__ frontier,
                   const int32_t* __restrict__ n_nodes, int F, int V, int k, int nmax, float kexp2,
                   double invT, RowTop* __restrict__ rows) {
    __shared__ float sv[kExpandMaxK][kTopThreads];
    __shared__ int si[kExpandMaxK][kTopThreads];
    __shared__ int head[kTopThreads];
    __shared__ float wm[kTopWaves], ws[kTopWaves];
    const int row = blockIdx.x, b = row / F;
    const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
    const int u = frontier[row], n = n_nodes[b];
    RowTop* out = rows + row;
    if (!(u >= 0 && u < min(n, nmax))) { // (workgroup-uniform) not a node: no row
        if (t == 0) out->count = 0;
        return;
    }
    const T* z = logits + static_cast<int64_t>(row) * V;

    // per-thread top-k, sorted (value desc, index asc); this thread's elements come in increasing
    // index order, so a strictly larger value is needed to enter
    float tv[kExpandMaxK];
    int ti[kExpandMaxK];
#pragma unroll
    for (int j = 0; j < kExpandMaxK; ++j) { tv[j] = -INFINITY; ti[j] = INT_MAX; }
    float thr = -INFINITY;               // the current k-th value (entry k-1) once k are held
    int held = 0;
    float m = -INFINITY, s = 0.f;        // online max and sum of exp2((x - m) kexp2)
    auto take = [&](float x, int xi) {
        const float mn = fmaxf(m, x);
        const float ref = (mn == -INFINITY) ? 0.f : mn;
        s = s * __builtin_amdgcn_exp2f((m - ref) * kexp2) + __builtin_amdgcn_exp2f((x - ref) * kexp2);
        m = mn;
        if (held < k || x > thr) {
            ++held;
            // insert: shift the worse entries down one place
            float cv = x;
            int ci = xi;
#pragma unroll
            for (int j = 0; j < kExpandMaxK; ++j) {
                const bool go = j < k && better(cv, ci, tv[j], ti[j]);
                const float ov = tv[j];
                const int oi = ti[j];
                tv[j] = go ? cv : ov;
                ti[j] = go ? ci : oi;
                cv = go ? ov : cv;
                ci = go ? oi : ci;
            }
            float nt = tv[0];
#pragma unroll
            for (int j = 1; j < kExpandMaxK; ++j) nt = (j == k - 1) ? tv[j] : nt;
            thr = nt;
        }
    };
    constexpr int kVec = Elem<T>::kVec;
    if ((V % kVec) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0) {
        for (int base = t * kVec; base < V; base += kTopThreads * kVec) {
            float x[kVec];
            Elem<T>::load_vec(z, base, x);
#pragma unroll
            for (int e = 0; e < kVec; ++e) take(x[e], base + e);
        }
    } else {
        for (int i = t; i < V; i += kTopThreads) take(Elem<T>::load(z, i), i);
    }

    // workgroup log-sum-exp (fp64 above the per-thread sums)
    wave_max_sum(m, s, kexp2);
    if (lane == 0) { wm[w] = m; ws[w] = s; }
#pragma unroll
    for (int j = 0; j < kExpandMaxK; ++j) { sv[j][t] = tv[j]; si[j][t] = ti[j]; }
    head[t] = 0;
    __syncthreads();
    if (w == 0) {
        // merge: k rounds, each taking the best head among the 256 sorted lists
        const int kk = min(k, V);
        for (int r = 0; r < kk; ++r) {
            float bv = -INFINITY;
            int bi = INT_MAX, bl = -1;
#pragma unroll
            for (int q = 0; q < kTopThreads / kWave; ++q) {
                const int l = q * kWave + lane;
                const int h = head[l];
                const float v = h < k ? sv[h][l] : -INFINITY;
                const int i = h < k ? si[h][l] : INT_MAX;
                if (i != INT_MAX && (bl < 0 || better(v, i, bv, bi))) { bv = v; bi = i; bl = l; }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float v2 = __shfl_xor(bv, o);
                const int i2 = __shfl_xor(bi, o), l2 = __shfl_xor(bl, o);
                if (l2 >= 0 && (bl < 0 || better(v2, i2, bv, bi))) { bv = v2; bi = i2; bl = l2; }
            }
            if (lane == 0 && bl >= 0) {
                out->tok[r] = bi;
                out->z[r] = bv;
                head[bl] += 1;
            }
            __builtin_amdgcn_s_waitcnt(0);   // (the head update is read by the next round)
            __builtin_amdgcn_wave_barrier();
        }
        if (lane == 0) {
            float M = -INFINITY;
            for (int q = 0; q < kTopWaves; ++q) M = fmaxf(M, wm[q]);
            double S = 0.0;
            for (int q = 0; q < kTopWaves; ++q)
                if (wm[q] != -INFINITY) S += static_cast<double>(ws[q]) * exp2(static_cast<double>(wm[q] - M) * kexp2);
            out->lse = static_cast<double>(M) * invT + log(S);
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
        if (j < r.count) sc = score[tb + frontier[b * F + f]] + (static_cast<double>(r.z[j]) * invT - r.lse);
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
            const int node = n + pos;
            parent[tb + node] = frontier[b * F + f];
            tokens[tb + node] = rb[f].tok[j];
            score[tb + node] = cs[c];
            new_frontier[static_cast<int64_t>(b) * keep + pos] = node;
        }
        done += all;
        __syncthreads();
    }
    for (int i = M + t; i < keep; i += kSelThreads) new_frontier[static_cast<int64_t>(b) * keep + i] = -1;
    if (t == 0) n_nodes[b] = n + M;
}

}  // namespace

size_t tree_expand_workspace_bytes(int B, int F) { return sizeof(RowTop) * static_cast<size_t>(B) * F; }

hipError_t launch_tree_expand(const TreeExpandArgs& a, hipStream_t stream) {
    RowTop* rows = static_cast<RowTop*>(a.workspace);
    const double invT = 1.0 / static_cast<double>(a.temperature);
    const float kexp2 = static_cast<float>(1.4426950408889634 * invT);
    if (a.bf16)
        hipLaunchKernelGGL(expand_topk_kernel<uint16_t>, dim3(a.B * a.F), dim3(kTopThreads), 0, stream,
                           static_cast<const uint16_t*>(a.logits), a.frontier, a.n_nodes, a.F, a.V, a.k, a.nmax,
                           kexp2, invT, rows);
    else
        hipLaunchKernelGGL(expand_topk_kernel<float>, dim3(a.B * a.F), dim3(kTopThreads), 0, stream,
                           static_cast<const float*>(a.logits), a.frontier, a.n_nodes, a.F, a.V, a.k, a.nmax,
                           kexp2, invT, rows);
    hipLaunchKernelGGL(expand_select_kernel, dim3(a.B), dim3(kSelThreads), 0, stream, rows, a.frontier, a.F, a.k,
                       a.keep, a.nmax, invT, a.parent, a.tokens, a.score, a.n_nodes, a.new_frontier);
    return hipGetLastError();
}

}  // namespace specv
