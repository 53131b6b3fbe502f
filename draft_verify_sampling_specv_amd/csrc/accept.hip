// Exact accept / reject / resample over the vocabulary.
//
// [SD-EAGLE] "The Exactness Rule", [SD-review] §2: p = softmax(target / T), q = softmax(draft / T);
// accept x if u < p(x)/q(x); at the first rejection draw from (p - q)+ and stop; if the whole path
// is accepted draw a bonus token from p of the last node; greedy at T = 0.  [PTD] Method 4,
// "Acceptance Logic": on a tree the children of a node are tested in index order as draws without
// replacement from q; after i rejections the target is (p - c_i q)+ / R_i (scalar form, see the
// walk below).
//
// Three launches on the caller's stream:
//   1. stats  grid (chunk, node, sequence): streams every target row and the draft rows of
//             internal nodes once, coalesced 16-byte loads, and writes per-chunk softmax
//             statistics (max, sum of exp) -- or (max, argmax) at T = 0.  This is the HBM-bound
//             pass; one exp per element.
//   2. walk   one 1024-thread workgroup per sequence: combines the chunk statistics, computes
//             p_tok / q_tok, runs the accept walk (all threads execute it in lock-step so that
//             the rare sibling-rejection passes over a row pair can use the whole workgroup),
//             and records the end node, the residual coefficient c and the draw uniform.
//   3. draw   grid (chunk, sequence): sums of the draw weights w(x) = (p(x) - c q(x))+ (c = 0 for
//             a bonus) per chunk of the end row; the last workgroup of a sequence to finish
//             (device-scope counter) scans the chunk sums, finds the chunk where the CDF crosses
//             u * W, and searches it.  Skipped at T = 0.
//
// Precision: per-element exponentials in fp32 (v_exp_f32), chunk sums in fp32, everything above
// chunk level (row normalisers, ratios, c, Q, R, the CDF threshold and the chunk prefix) in fp64.

#include "common.h"
#include "kernels.h"

namespace specv {

namespace {

constexpr int kStatThreads = 256;
constexpr int kUnroll = 4;
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / kWave;

template <typename T>
constexpr int chunk_elems() {
    return kStatThreads * Elem<T>::kVec * kUnroll;   // bf16: 8192, fp32: 4096 (16 KB per row)
}

struct WalkResult {        // per sequence: what the draw kernel must sample
    int32_t mode;          // 0: nothing to draw (greedy or invalid sequence); 1: draw
    int32_t row;           // end node
    float m_t, m_d;        // raw-logit maxima of the end node's target / draft rows
    float p_scale;         // 1 / S_t
    float q_scale;         // c / S_d   (0: bonus, weights are p itself)
    double u;              // draw uniform
};
static_assert(sizeof(WalkResult) == 32, "WalkResult layout");

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct AcceptLayout {
    size_t stats, res, sums, counters, total;
    AcceptLayout(int B, int n1, int nchunk) {
        stats = 0;
        res = align256(stats + sizeof(float4) * size_t(B) * n1 * nchunk);
        sums = align256(res + sizeof(WalkResult) * size_t(B));
        counters = align256(sums + sizeof(float) * size_t(B) * nchunk);
        total = align256(counters + sizeof(uint32_t) * size_t(B));
    }
};

// Load this thread's share of [lo, hi) of one row: kUnroll vectors of kVec contiguous elements,
// vector u at lo + (u * kStatThreads + t) * kVec.  Out-of-range elements read as -inf.
template <typename T, bool kVecOK>
__device__ __forceinline__ void load_chunk(const T* __restrict__ row, int lo, int hi, int t,
                                           float* out) {
    constexpr int kVec = Elem<T>::kVec;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int base = lo + (u * kStatThreads + t) * kVec;
        if (kVecOK && base + kVec <= hi) {
            Elem<T>::load_vec(row, base, out + u * kVec);
        } else {
#pragma unroll
            for (int e = 0; e < kVec; ++e)
                out[u * kVec + e] = (base + e < hi) ? Elem<T>::load(row, base + e) : -INFINITY;
        }
    }
}

// Draw weight of one element: (p(x) - c q(x))+ with p = exp2((zt - mt) k) / S_t etc.
__device__ __forceinline__ float draw_weight(float zt, float zd, float mt, float md, float k,
                                             float p_scale, float q_scale) {
    float p = __builtin_amdgcn_exp2f((zt - mt) * k) * p_scale;
    float q = __builtin_amdgcn_exp2f((zd - md) * k) * q_scale;
    return fmaxf(p - q, 0.0f);
}

template <int kThreads>
__device__ double block_sum(double x, double* red) {
    x = wave_sum(x);
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    __syncthreads();
    if (lane == 0) red[w] = x;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) s += red[i];
    return s;
}

// ------------------------------------------------------------------------------------ 1. stats

template <typename T, bool kGreedy, bool kVecOK>
__global__ void __launch_bounds__(kStatThreads)
accept_stats_kernel(const T* __restrict__ target, const T* __restrict__ draft,
                    const int32_t* __restrict__ parent, int n1, int V, int nchunk, float k,
                    float4* __restrict__ stats) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int CH = chunk_elems<T>();
    const int c = blockIdx.x, v = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x;
    const int w = t / kWave, lane = t % kWave;
    const int64_t row = (static_cast<int64_t>(b) * n1 + v) * V;
    const int lo = c * CH;
    const int hi = min(V, lo + CH);
    __shared__ float4 part[kStatThreads / kWave];

    float zt[kUnroll * kVec];
    load_chunk<T, kVecOK>(target + row, lo, hi, t, zt);

    if (kGreedy) {
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const int idx = lo + (u * kStatThreads + t) * kVec + e;
                if (idx < hi) argmax_merge(bv, bi, zt[u * kVec + e], idx);
            }
        wave_argmax(bv, bi);
        if (lane == 0) part[w] = make_float4(bv, __int_as_float(bi), 0.f, 0.f);
        __syncthreads();
        if (t == 0) {
            float fv = part[0].x;
            int fi = __float_as_int(part[0].y);
            for (int i = 1; i < kStatThreads / kWave; ++i)
                argmax_merge(fv, fi, part[i].x, __float_as_int(part[i].y));
            stats[(static_cast<int64_t>(b) * n1 + v) * nchunk + c] =
                make_float4(fv, __int_as_float(fi), 0.f, 0.f);
        }
        return;
    }

    // Draft rows are read only for internal nodes (a leaf's draft row proposes nothing).
    int found = 0;
    const int32_t* pb = parent + static_cast<int64_t>(b) * n1;
    for (int i = v + 1 + t; i < n1; i += kStatThreads) found |= (pb[i] == v);
    const bool want_draft = __syncthreads_or(found) != 0;

    float zd[kUnroll * kVec];
    if (want_draft) load_chunk<T, kVecOK>(draft + row, lo, hi, t, zd);

    float mt = -INFINITY, st = 0.f;
#pragma unroll
    for (int e = 0; e < kUnroll * kVec; ++e) mt = fmaxf(mt, zt[e]);
    if (mt != -INFINITY) {
#pragma unroll
        for (int e = 0; e < kUnroll * kVec; ++e) st += __builtin_amdgcn_exp2f((zt[e] - mt) * k);
    }
    float md = -INFINITY, sd = 0.f;
    if (want_draft) {
#pragma unroll
        for (int e = 0; e < kUnroll * kVec; ++e) md = fmaxf(md, zd[e]);
        if (md != -INFINITY) {
#pragma unroll
            for (int e = 0; e < kUnroll * kVec; ++e) sd += __builtin_amdgcn_exp2f((zd[e] - md) * k);
        }
    }
    wave_max_sum(mt, st, k);
    if (want_draft) wave_max_sum(md, sd, k);
    if (lane == 0) part[w] = make_float4(mt, st, md, sd);
    __syncthreads();
    if (t == 0) {
        float4 r = part[0];
        for (int i = 1; i < kStatThreads / kWave; ++i) {
            merge_max_sum(r.x, r.y, part[i].x, part[i].y, k);
            merge_max_sum(r.z, r.w, part[i].z, part[i].w, k);
        }
        stats[(static_cast<int64_t>(b) * n1 + v) * nchunk + c] = r;
    }
}

// ------------------------------------------------------------------------------------ 2. walk

// Sum over the vocabulary of (p(x) - c q(x))+ for row v: the residual mass R(c).  Whole workgroup.
template <typename T, bool kVecOK>
__device__ double residual_mass(const T* __restrict__ trow, const T* __restrict__ drow, int V,
                                float mt, float md, float k, float p_scale, float q_scale,
                                double* red) {
    constexpr int kVec = Elem<T>::kVec;
    float acc = 0.f;
    float zt[kVec], zd[kVec];
    for (int base = threadIdx.x * kVec; base < V; base += kWalkThreads * kVec) {
        if (kVecOK) {
            Elem<T>::load_vec(trow, base, zt);
            Elem<T>::load_vec(drow, base, zd);
        } else {
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                zt[e] = (base + e < V) ? Elem<T>::load(trow, base + e) : -INFINITY;
                zd[e] = (base + e < V) ? Elem<T>::load(drow, base + e) : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc += draw_weight(zt[e], zd[e], mt, md, k, p_scale, q_scale);
    }
    return block_sum<kWalkThreads>(static_cast<double>(acc), red);
}

// Is there a child of v with index in (after, n1)?  Uniform over the wave.
__device__ __forceinline__ bool has_child_after(const int32_t* par, int n1, int v, int after) {
    const int lane = threadIdx.x % kWave;
    for (int base = (after + 1) & ~(kWave - 1); base < n1; base += kWave) {
        const int i = base + lane;
        if (__ballot(i > after && i < n1 && par[i] == v)) return true;
    }
    return false;
}

// Does an earlier sibling (index < ch) of ch carry token x?
__device__ __forceinline__ bool earlier_sibling_has(const int32_t* par, const int32_t* tok, int v,
                                                    int ch, int x) {
    const int lane = threadIdx.x % kWave;
    for (int base = (v + 1) & ~(kWave - 1); base < ch; base += kWave) {
        const int i = base + lane;
        if (__ballot(i > v && i < ch && par[i] == v && tok[i] == x)) return true;
    }
    return false;
}

template <typename T, bool kGreedy, bool kVecOK>
__global__ void __launch_bounds__(kWalkThreads)
accept_walk_kernel(const T* __restrict__ target, const T* __restrict__ draft,
                   const int32_t* __restrict__ tokens, const int32_t* __restrict__ parent, int n1,
                   int V, int nchunk, float k, double invT, uint64_t seed, uint64_t offset,
                   const float4* __restrict__ stats, WalkResult* __restrict__ res,
                   uint32_t* __restrict__ counters, int32_t* __restrict__ accept_len,
                   int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_nodes,
                   float* __restrict__ p_tok, float* __restrict__ q_tok) {
    __shared__ int32_t par[kMaxNodes];
    __shared__ int32_t tok[kMaxNodes];
    __shared__ int32_t haskid[kMaxNodes];
    __shared__ float Mt[kMaxNodes], Md[kMaxNodes];
    __shared__ double St[kMaxNodes], Sd[kMaxNodes];
    __shared__ int32_t amax[kMaxNodes];
    __shared__ double red[kWalkWaves];
    __shared__ int bad;

    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int w = t / kWave, lane = t % kWave;
    const int64_t seq = static_cast<int64_t>(b) * n1;

    // -- stage and validate the parent array and the draft tokens
    if (t == 0) bad = 0;
    for (int i = t; i < n1; i += kWalkThreads) haskid[i] = 0;
    __syncthreads();
    for (int i = t; i < n1; i += kWalkThreads) {
        const int p = parent[seq + i];
        const int x = tokens[seq + i];
        par[i] = p;
        tok[i] = x;
        const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i && x >= 0 && x < V);
        if (!ok) bad = 1;
    }
    __syncthreads();
    if (bad) {
        for (int i = t; i < n1; i += kWalkThreads) {
            out_tokens[seq + i] = -1;
            out_nodes[seq + i] = -1;
            if (p_tok) p_tok[seq + i] = NAN;
            if (q_tok) q_tok[seq + i] = NAN;
        }
        if (t == 0) {
            accept_len[b] = -1;
            res[b].mode = 0;
        }
        return;
    }
    for (int i = 1 + t; i < n1; i += kWalkThreads) haskid[par[i]] = 1;
    __syncthreads();

    // -- combine chunk statistics per row (one wave per row, lanes over chunks)
    for (int v = w; v < n1; v += kWalkWaves) {
        const float4* sv = stats + (seq + v) * nchunk;
        if (kGreedy) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            for (int c = lane; c < nchunk; c += kWave) {
                float4 s = sv[c];
                argmax_merge(bv, bi, s.x, __float_as_int(s.y));
            }
            wave_argmax(bv, bi);
            if (lane == 0) amax[v] = (bi >= 0 && bi < V) ? bi : 0;
        } else {
            const bool dr = haskid[v] != 0;
            float mt = -INFINITY, md = -INFINITY;
            for (int c = lane; c < nchunk; c += kWave) {
                float4 s = sv[c];
                mt = fmaxf(mt, s.x);
                if (dr) md = fmaxf(md, s.z);
            }
            mt = wave_max(mt);
            md = wave_max(md);
            double st = 0.0, sd = 0.0;
            for (int c = lane; c < nchunk; c += kWave) {
                float4 s = sv[c];
                if (s.x != -INFINITY) st += static_cast<double>(s.y) * exp2(static_cast<double>((s.x - mt) * k));
                if (dr && s.z != -INFINITY) sd += static_cast<double>(s.w) * exp2(static_cast<double>((s.z - md) * k));
            }
            st = wave_sum(st);
            sd = wave_sum(sd);
            if (lane == 0) {
                Mt[v] = mt; St[v] = st;
                Md[v] = md; Sd[v] = sd;
            }
        }
    }
    __syncthreads();

    // -- p_tok / q_tok: target and draft probability of every draft token under its parent's row
    if (p_tok || q_tok) {
        for (int v = t; v < n1; v += kWalkThreads) {
            float pv = NAN, qv = NAN;
            if (!kGreedy && v > 0) {
                const int pa = par[v], x = tok[v];
                const double zt = Elem<T>::load(target + (seq + pa) * V, x);
                const double zd = Elem<T>::load(draft + (seq + pa) * V, x);
                pv = static_cast<float>(exp((zt - Mt[pa]) * invT) / St[pa]);
                qv = static_cast<float>(exp((zd - Md[pa]) * invT) / Sd[pa]);
            }
            if (p_tok) p_tok[seq + v] = pv;
            if (q_tok) q_tok[seq + v] = qv;
        }
    }

    // -- the walk: executed identically by every thread (uniform control flow)
    int v = 0, n = 0;
    double cs = 0.0;
    while (true) {
        int accepted = -1;
        if (kGreedy) {
            const int y = amax[v];
            for (int base = (v + 1) & ~(kWave - 1); base < n1 && accepted < 0; base += kWave) {
                const int i = base + lane;
                const uint64_t m = __ballot(i > v && i < n1 && par[i] == v && tok[i] == y);
                if (m) accepted = base + __ffsll(static_cast<unsigned long long>(m)) - 1;
            }
        } else {
            cs = 0.0;
            double R = 1.0, Q = 1.0;
            const int64_t rv = (seq + v) * V;
            for (int base = (v + 1) & ~(kWave - 1); base < n1 && accepted < 0; base += kWave) {
                const int i = base + lane;
                uint64_t m = __ballot(i > v && i < n1 && par[i] == v);
                while (m && accepted < 0) {
                    const int ch = base + __ffsll(static_cast<unsigned long long>(m)) - 1;
                    m &= m - 1;
                    const int x = tok[ch];
                    if (earlier_sibling_has(par, tok, v, ch, x)) continue;
                    const double zt = Elem<T>::load(target + rv, x);
                    const double zd = Elem<T>::load(draft + rv, x);
                    const double lp = (zt - Mt[v]) * invT;
                    const double lq = (zd - Md[v]) * invT;
                    const double pq = exp(lp - lq) * (Sd[v] / St[v]);
                    const double qx = exp(lq) / Sd[v];
                    const double ratio = fmax(0.0, pq - cs) * Q / R;
                    const U64x4 rnd = philox4x64_10(static_cast<uint64_t>(ch), static_cast<uint64_t>(b),
                                                    offset, 0, seed, 0);
                    if (word_to_uniform(rnd.w[0]) < ratio) {
                        accepted = ch;
                        break;
                    }
                    // rejection: c <- c + R/Q, Q <- Q - q(x), R <- R(c) if another sibling follows
                    const double cn = cs + R / Q;
                    Q -= qx;
                    if (has_child_after(par, n1, v, ch)) {
                        const double Rn = residual_mass<T, kVecOK>(
                            target + rv, draft + rv, V, Mt[v], Md[v], k,
                            static_cast<float>(1.0 / St[v]), static_cast<float>(cn / Sd[v]), red);
                        if (Rn > 0.0) {
                            cs = cn;
                            R = Rn;
                        }
                    } else {
                        cs = cn;
                    }
                }
            }
        }
        if (accepted < 0) break;
        if (t == 0) {
            out_nodes[seq + n] = accepted;
            out_tokens[seq + n] = tok[accepted];
        }
        ++n;
        v = accepted;
    }

    // -- record the outcome
    for (int i = n + t; i < n1; i += kWalkThreads) {
        out_nodes[seq + i] = -1;
        if (i > n) out_tokens[seq + i] = -1;
    }
    if (t == 0) {
        accept_len[b] = n;
        if (kGreedy) {
            out_tokens[seq + n] = amax[v];
            res[b].mode = 0;
        } else {
            const U64x4 rnd = philox4x64_10(static_cast<uint64_t>(v), static_cast<uint64_t>(b),
                                            offset, 0, seed, 0);
            WalkResult r;
            r.mode = 1;
            r.row = v;
            r.m_t = Mt[v];
            r.m_d = (cs > 0.0) ? Md[v] : 0.f;
            r.p_scale = static_cast<float>(1.0 / St[v]);
            r.q_scale = (cs > 0.0) ? static_cast<float>(cs / Sd[v]) : 0.f;
            r.u = word_to_uniform(rnd.w[1]);
            res[b] = r;
            counters[b] = 0;
        }
    }
}

// ------------------------------------------------------------------------------------ 3. draw

template <typename T, bool kVecOK>
__global__ void __launch_bounds__(kStatThreads)
accept_draw_kernel(const T* __restrict__ target, const T* __restrict__ draft, int n1, int V,
                   int nchunk, float k, const WalkResult* __restrict__ res,
                   float* __restrict__ chunk_sums, uint32_t* __restrict__ counters,
                   const int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int CH = chunk_elems<T>();
    constexpr int kPer = kUnroll * kVec;
    constexpr int kWaves = kStatThreads / kWave;
    const int c = blockIdx.x, b = blockIdx.y;
    const int t = threadIdx.x;
    const int w = t / kWave, lane = t % kWave;
    const WalkResult r = res[b];
    if (r.mode == 0) return;

    const int64_t row = (static_cast<int64_t>(b) * n1 + r.row) * V;
    const bool use_q = r.q_scale != 0.f;
    __shared__ double red[kWaves];
    __shared__ int last;

    {
        const int lo = c * CH, hi = min(V, lo + CH);
        float zt[kPer], zd[kPer];
        load_chunk<T, kVecOK>(target + row, lo, hi, t, zt);
        if (use_q) load_chunk<T, kVecOK>(draft + row, lo, hi, t, zd);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            acc += draw_weight(zt[e], use_q ? zd[e] : 0.f, r.m_t, r.m_d, k, r.p_scale, r.q_scale);
        const double s = block_sum<kStatThreads>(static_cast<double>(acc), red);
        if (t == 0) {
            chunk_sums[static_cast<int64_t>(b) * nchunk + c] = static_cast<float>(s);
            __threadfence();
            last = (atomicAdd(&counters[b], 1u) == static_cast<uint32_t>(nchunk - 1));
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
    }

    // ---- the last workgroup of this sequence samples
    __shared__ float wbuf[CH];
    __shared__ int sel_chunk;
    __shared__ double sel_base, thresh;
    __shared__ int found;
    const float* sums = chunk_sums + static_cast<int64_t>(b) * nchunk;

    if (w == 0) {
        // chunk totals: lane l owns a contiguous group of chunks; fp64 inclusive scan over lanes
        const int g = (nchunk + kWave - 1) / kWave;
        const int c0 = min(nchunk, lane * g), c1 = min(nchunk, c0 + g);
        double gs = 0.0;
        for (int i = c0; i < c1; ++i) gs += __hip_atomic_load(&sums[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        double incl = gs;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const double y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const double total = __shfl(incl, kWave - 1);
        const double tt = r.u * total;
        const uint64_t m = __ballot(c1 > c0 && incl > tt);
        int chosen = -1;
        double base = 0.0;
        if (total > 0.0) {
            int L;
            if (m) {
                L = __ffsll(static_cast<unsigned long long>(m)) - 1;
            } else {   // rounding put u*W at or above the total: take the last group with mass
                const uint64_t nz = __ballot(gs > 0.0);
                L = 63 - __clzll(static_cast<long long>(nz));
            }
            if (lane == L) {
                double acc = incl - gs;
                int lastpos = -1;
                double lastbase = acc;
                for (int i = c0; i < c1; ++i) {
                    const double s = __hip_atomic_load(&sums[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (s > 0.0) { lastpos = i; lastbase = acc; }
                    if (acc + s > tt) { chosen = i; base = acc; break; }
                    acc += s;
                }
                if (chosen < 0) { chosen = lastpos; base = lastbase; }
            }
            chosen = __shfl(chosen, L);
            base = __shfl(base, L);
        }
        if (lane == 0) {
            sel_chunk = chosen;
            sel_base = base;
            thresh = tt;
            found = INT_MAX;
        }
    }
    __syncthreads();

    int y = -1;
    if (sel_chunk >= 0) {
        // recompute the weights of the chosen chunk in index order and search it
        const int lo = sel_chunk * CH, hi = min(V, lo + CH);
        float zt[kPer], zd[kPer];
        load_chunk<T, kVecOK>(target + row, lo, hi, t, zt);
        if (use_q) load_chunk<T, kVecOK>(draft + row, lo, hi, t, zd);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const int off = (u * kStatThreads + t) * kVec + e;
                wbuf[off] = draw_weight(zt[u * kVec + e], use_q ? zd[u * kVec + e] : 0.f, r.m_t,
                                        r.m_d, k, r.p_scale, r.q_scale);
            }
        __syncthreads();
        // thread t scans the contiguous segment [t*kPer, (t+1)*kPer)
        float seg[kPer];
        float ssum = 0.f;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            seg[e] = wbuf[t * kPer + e];
            ssum += seg[e];
        }
        // exclusive scan of segment sums in thread order (fp64)
        double incl = ssum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const double yv = __shfl_up(incl, o);
            if (lane >= o) incl += yv;
        }
        __syncthreads();
        if (lane == kWave - 1) red[w] = incl;
        __syncthreads();
        double before = 0.0;
        for (int i = 0; i < w; ++i) before += red[i];
        double acc = sel_base + before + (incl - ssum);
        int cand = INT_MAX;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            acc += seg[e];
            if (cand == INT_MAX && seg[e] > 0.f && acc > thresh) cand = lo + t * kPer + e;
        }
        if (cand != INT_MAX) atomicMin(&found, cand);
        __syncthreads();
        y = found;
        if (y == INT_MAX || y >= hi) {
            // rounding kept the threshold above this chunk's running sum: last positive element
            int lastpos = -1;
            for (int e = kPer - 1; e >= 0; --e)
                if (seg[e] > 0.f) { lastpos = lo + t * kPer + e; break; }
            __syncthreads();
            if (t == 0) found = -1;
            __syncthreads();
            if (lastpos >= 0 && lastpos < hi) atomicMax(&found, lastpos);
            __syncthreads();
            y = found;
        }
    }
    if (y < 0) {
        // no residual mass at all (a zero-probability event in exact arithmetic): emit the token
        // with the largest p(x) - c q(x), lowest index on ties
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int base = t; base < V; base += kStatThreads) {
            const float zt = Elem<T>::load(target + row, base);
            const float zd = use_q ? Elem<T>::load(draft + row, base) : 0.f;
            const float d = __builtin_amdgcn_exp2f((zt - r.m_t) * k) * r.p_scale -
                            __builtin_amdgcn_exp2f((zd - r.m_d) * k) * r.q_scale;
            argmax_merge(bv, bi, d, base);
        }
        wave_argmax(bv, bi);
        __shared__ float pv[kWaves];
        __shared__ int pi[kWaves];
        if (lane == 0) { pv[w] = bv; pi[w] = bi; }
        __syncthreads();
        if (t == 0) {
            for (int i = 1; i < kWaves; ++i) argmax_merge(pv[0], pi[0], pv[i], pi[i]);
            found = (pi[0] >= 0 && pi[0] < V) ? pi[0] : 0;
        }
        __syncthreads();
        y = found;
    }
    if (t == 0) out_tokens[static_cast<int64_t>(b) * n1 + accept_len[b]] = y;
}

template <typename T, bool kVecOK>
hipError_t launch_typed(const AcceptArgs& a, hipStream_t stream) {
    constexpr int CH = chunk_elems<T>();
    const int nchunk = (a.V + CH - 1) / CH;
    const AcceptLayout lay(a.B, a.n1, nchunk);
    char* ws = static_cast<char*>(a.workspace);
    float4* stats = reinterpret_cast<float4*>(ws + lay.stats);
    WalkResult* res = reinterpret_cast<WalkResult*>(ws + lay.res);
    float* sums = reinterpret_cast<float*>(ws + lay.sums);
    uint32_t* counters = reinterpret_cast<uint32_t*>(ws + lay.counters);
    const T* target = static_cast<const T*>(a.target);
    const T* draft = static_cast<const T*>(a.draft);
    const bool greedy = a.temperature == 0.f;
    const double invT = greedy ? 0.0 : 1.0 / static_cast<double>(a.temperature);
    const float k = greedy ? 0.f : static_cast<float>(1.4426950408889634 * invT);   // log2(e) / T

    const dim3 sgrid(nchunk, a.n1, a.B);
    if (greedy) {
        hipLaunchKernelGGL((accept_stats_kernel<T, true, kVecOK>), sgrid, dim3(kStatThreads), 0, stream,
                           target, draft, a.parent, a.n1, a.V, nchunk, k, stats);
        hipLaunchKernelGGL((accept_walk_kernel<T, true, kVecOK>), dim3(a.B), dim3(kWalkThreads), 0, stream,
                           target, draft, a.tokens, a.parent, a.n1, a.V, nchunk, k, invT, a.seed,
                           a.offset, stats, res, counters, a.accept_len, a.out_tokens, a.out_nodes,
                           a.p_tok, a.q_tok);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((accept_stats_kernel<T, false, kVecOK>), sgrid, dim3(kStatThreads), 0, stream,
                       target, draft, a.parent, a.n1, a.V, nchunk, k, stats);
    hipLaunchKernelGGL((accept_walk_kernel<T, false, kVecOK>), dim3(a.B), dim3(kWalkThreads), 0, stream,
                       target, draft, a.tokens, a.parent, a.n1, a.V, nchunk, k, invT, a.seed, a.offset,
                       stats, res, counters, a.accept_len, a.out_tokens, a.out_nodes, a.p_tok, a.q_tok);
    hipLaunchKernelGGL((accept_draw_kernel<T, kVecOK>), dim3(nchunk, a.B), dim3(kStatThreads), 0, stream,
                       target, draft, a.n1, a.V, nchunk, k, res, sums, counters, a.accept_len,
                       a.out_tokens);
    return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

size_t accept_workspace_bytes(int B, int n1, int V, bool bf16) {
    const int CH = bf16 ? chunk_elems<uint16_t>() : chunk_elems<float>();
    const int nchunk = (V + CH - 1) / CH;
    return AcceptLayout(B, n1, nchunk).total;
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
    const bool vec = aligned16(a.target) && (a.draft == nullptr || aligned16(a.draft));
    if (a.bf16) {
        if (vec && a.V % Elem<uint16_t>::kVec == 0) return launch_typed<uint16_t, true>(a, stream);
        return launch_typed<uint16_t, false>(a, stream);
    }
    if (vec && a.V % Elem<float>::kVec == 0) return launch_typed<float, true>(a, stream);
    return launch_typed<float, false>(a, stream);
}

}  // namespace specv
