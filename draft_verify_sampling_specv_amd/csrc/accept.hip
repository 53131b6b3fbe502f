// Exact accept / reject / resample over the vocabulary.
//
// [SD-EAGLE] "The Exactness Rule", [SD-review] §2: p = softmax(target / T), q = softmax(draft / T);
// accept x if u < p(x)/q(x); at the first rejection draw from (p - q)+ and stop; if the whole path
// is accepted draw a bonus token from p of the last node; greedy at T = 0.  [PTD] Method 4,
// "Acceptance Logic": on a tree the children of a node are tested in index order as draws without
// replacement from q; after i rejections the target is (p - c_i q)+ / R_i (scalar form, see the
// walk below).
//
// Two launches on the caller's stream:
//   1. stats   grid (chunk, node, sequence): streams every target row and the draft rows of
//              internal nodes once, coalesced 16-byte loads, and writes per-chunk softmax
//              statistics (max, sum of exp) -- or (max, argmax) at T = 0.  This is the HBM-bound
//              pass; one exp per element.
//   2. finish  one 1024-thread workgroup per sequence: combines the chunk statistics; computes,
//              for every draft node in parallel, p and q of its token under its parent's rows,
//              the ratio p/q and its acceptance uniform; one wave then runs the walk (scalar, from
//              those tables); the rare sibling-rejection passes R(c) = sum (p - c q)+ over a row
//              pair and the final draw pass use the whole workgroup.  The draw pass records the
//              sum of every 64*kVec-element segment in LDS; the segment holding the CDF crossing
//              is found by a block scan and searched by one wave.
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
constexpr int kMaxVocab = 1 << 21;
constexpr double kAllDraftBytes = 32.0 * (1 << 20);   // target logits of a call

template <typename T>
constexpr int chunk_elems() {
    return kStatThreads * Elem<T>::kVec * kUnroll;   // bf16: 8192, fp32: 4096 (16 KB per row)
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct AcceptLayout {
    size_t stats, total;
    AcceptLayout(int B, int n1, int nchunk) {
        stats = 0;
        total = align256(stats + sizeof(float4) * size_t(B) * n1 * nchunk);
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

// ------------------------------------------------------------------------------------ 1. stats

template <typename T, bool kGreedy, bool kVecOK, bool kAllDraft>
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

    // Draft rows are needed only for internal nodes (a leaf's draft row proposes nothing).  Small
    // calls (kAllDraft) read every draft row instead: one dependent round trip to the parent
    // array costs more there than the leaf rows' bytes.
    bool want_draft = true;
    if (!kAllDraft) {
        int found = 0;
        const int32_t* pb = parent + static_cast<int64_t>(b) * n1;
        for (int i = v + 1 + t; i < n1; i += kStatThreads) found |= (pb[i] == v);
        want_draft = __syncthreads_or(found) != 0;
    }

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

// ------------------------------------------------------------------------------------ 2. finish

// Streaming pass over one row pair with the draw weights w(x) = (p(x) - c q(x))+ (c = q_scale S_d;
// q_scale == 0: w = p).  Tile i covers kWalkThreads * kVec consecutive elements; within a tile
// wave ww owns the contiguous segment of 64 * kVec elements starting at (ww * 64) * kVec.  The
// segment sums are written to seg[i * kWalkWaves + ww] (index order) if seg != nullptr.  Loads of
// up to kPassBatch tiles are issued together so that their latencies overlap.
// Returns the total (fp64, identical in all threads).
constexpr int kPassBatch = 4;

template <typename T>
__device__ __forceinline__ void cvt_vec(const uint4& r, float* out);
template <>
__device__ __forceinline__ void cvt_vec<float>(const uint4& r, float* out) {
    out[0] = __uint_as_float(r.x); out[1] = __uint_as_float(r.y);
    out[2] = __uint_as_float(r.z); out[3] = __uint_as_float(r.w);
}
template <>
__device__ __forceinline__ void cvt_vec<uint16_t>(const uint4& r, float* out) {
    out[0] = bf16_lo(r.x); out[1] = bf16_hi(r.x); out[2] = bf16_lo(r.y); out[3] = bf16_hi(r.y);
    out[4] = bf16_lo(r.z); out[5] = bf16_hi(r.z); out[6] = bf16_lo(r.w); out[7] = bf16_hi(r.w);
}

template <typename T, bool kVecOK>
__device__ __forceinline__ void load_pair(const T* __restrict__ trow, const T* __restrict__ drow, int V,
                                          int base, bool use_q, float* zt, float* zd) {
    constexpr int kVec = Elem<T>::kVec;
    if (kVecOK && base + kVec <= V) {
        Elem<T>::load_vec(trow, base, zt);
        if (use_q) Elem<T>::load_vec(drow, base, zd);
    } else {
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            zt[e] = (base + e < V) ? Elem<T>::load(trow, base + e) : -INFINITY;
            zd[e] = (use_q && base + e < V) ? Elem<T>::load(drow, base + e) : -INFINITY;
        }
    }
    if (!use_q) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) zd[e] = -INFINITY;
    }
}

template <typename T, bool kVecOK>
__device__ double row_pass(const T* __restrict__ trow, const T* __restrict__ drow, int V, float mt,
                           float md, float k, float p_scale, float q_scale, float* seg, double* red,
                           uint4 (&rt)[kPassBatch], uint4 (&rd)[kPassBatch]) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int kTile = kWalkThreads * kVec;
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const bool use_q = q_scale != 0.f;
    double acc = 0.0;
    const int ntile = (V + kTile - 1) / kTile;
    for (int i0 = 0; i0 < ntile; i0 += kPassBatch) {
        if (kVecOK) {
#pragma unroll
            for (int j = 0; j < kPassBatch; ++j) {
                const int base = (i0 + j) * kTile + threadIdx.x * kVec;
                rt[j] = make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
                rd[j] = rt[j];
                if (i0 + j < ntile && base < V) {
                    rt[j] = *reinterpret_cast<const uint4*>(trow + base);
                    if (use_q) rd[j] = *reinterpret_cast<const uint4*>(drow + base);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kPassBatch; ++j) {
            if (i0 + j >= ntile) break;
            const int base = (i0 + j) * kTile + threadIdx.x * kVec;
            float zt[kVec], zd[kVec];
            if (kVecOK) {
                if (base < V) {
                    cvt_vec<T>(rt[j], zt);
                    if (use_q) cvt_vec<T>(rd[j], zd);
                }
                if (!(base < V) || !use_q) {
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        zd[e] = -INFINITY;
                        if (!(base < V)) zt[e] = -INFINITY;
                    }
                }
            } else {
                load_pair<T, false>(trow, drow, V, base, use_q, zt, zd);
            }
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < kVec; ++e) sum += draw_weight(zt[e], zd[e], mt, md, k, p_scale, q_scale);
            sum = wave_sum(sum);
            if (seg && lane == 0) seg[(i0 + j) * kWalkWaves + w] = sum;
            acc += sum;
        }
    }
    // every lane of a wave holds the same acc: add the wave totals
    __syncthreads();
    if (lane == 0) red[w] = acc;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < kWalkWaves; ++i) tot += red[i];
    return tot;
}

template <typename T, bool kGreedy, bool kVecOK>
__global__ void __launch_bounds__(kWalkThreads)
accept_finish_kernel(const T* __restrict__ target, const T* __restrict__ draft,
                     const int32_t* __restrict__ tokens, const int32_t* __restrict__ parent, int n1,
                     int V, int nchunk, float k, double invT, uint64_t seed, uint64_t offset,
                     const float4* __restrict__ stats, int32_t* __restrict__ accept_len,
                     int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_nodes,
                     float* __restrict__ p_tok, float* __restrict__ q_tok) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int kTile = kWalkThreads * kVec;
    constexpr int kMaxSeg = (kMaxVocab + kTile - 1) / kTile * kWalkWaves;
    __shared__ int32_t par[kMaxNodes];
    __shared__ int32_t tok[kMaxNodes];
    __shared__ int32_t info[kMaxNodes];     // greedy: argmax token of the row; else: has children
    __shared__ int32_t fch[kMaxNodes];      // first child (n1 if none)
    __shared__ int32_t nsib[kMaxNodes];     // next sibling (-1 if none)
    __shared__ int32_t dup[kMaxNodes];      // token repeats an earlier sibling's
    __shared__ float Mt[kMaxNodes], Md[kMaxNodes];
    __shared__ double St[kMaxNodes], Sd[kMaxNodes];
    __shared__ double pq[kMaxNodes];        // p(x)/q(x) of node x under its parent's rows
    __shared__ float qx[kMaxNodes];         // q(x)
    __shared__ double uacc[kMaxNodes];      // acceptance uniforms
    __shared__ double ures[kMaxNodes];      // draw uniforms
    __shared__ int32_t path[kMaxNodes];
    __shared__ float seg[kMaxSeg];
    __shared__ double red[kWalkWaves];
    __shared__ int s_bad, s_cmd, s_row, s_n, s_sel, s_found;
    __shared__ float s_ps, s_qs;
    __shared__ double s_R, s_base;

    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int w = t / kWave, lane = t % kWave;
    const int64_t seq = static_cast<int64_t>(b) * n1;

    // -- A. issue the independent loads first: the sequence's chunk statistics (staged in LDS when
    //       they fit), the parent array and the draft tokens; validate
    __shared__ float4 sst[kWalkThreads];
    const bool stage = n1 * nchunk <= kWalkThreads;
    float4 mystat = make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
    if (stage && t < n1 * nchunk) mystat = stats[seq * nchunk + t];
    if (t == 0) s_bad = 0;
    for (int i = t; i < n1; i += kWalkThreads) {
        info[i] = 0;
        fch[i] = n1;
    }
    __syncthreads();
    for (int i = t; i < n1; i += kWalkThreads) {
        const int p = parent[seq + i];
        const int x = tokens[seq + i];
        par[i] = p;
        tok[i] = x;
        const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i && x >= 0 && x < V);
        if (!ok) s_bad = 1;
    }
    if (stage) sst[t] = mystat;
    __syncthreads();
    if (s_bad) {
        for (int i = t; i < n1; i += kWalkThreads) {
            out_tokens[seq + i] = -1;
            out_nodes[seq + i] = -1;
            if (p_tok) p_tok[seq + i] = NAN;
            if (q_tok) q_tok[seq + i] = NAN;
        }
        if (t == 0) accept_len[b] = -1;
        return;
    }

    // -- B. gather every draft token's logits under its parent's rows (in flight during the
    //       combine); tree links: first child, next sibling, repeated sibling tokens
    float gzt = 0.f, gzd = 0.f;
    if (!kGreedy && t > 0 && t < n1) {
        const int pa = par[t], x = tok[t];
        gzt = Elem<T>::load(target + (seq + pa) * V, x);
        gzd = Elem<T>::load(draft + (seq + pa) * V, x);
    }
    for (int c = 1 + t; c < n1; c += kWalkThreads) {
        const int pa = par[c], x = tok[c];
        if (!kGreedy) info[pa] = 1;
        atomicMin(&fch[pa], c);
        int nx = -1;
        for (int i = c + 1; i < n1; ++i)
            if (par[i] == pa) { nx = i; break; }
        nsib[c] = nx;
        int d = 0;
        for (int i = c - 1; i > pa; --i)
            if (par[i] == pa && tok[i] == x) { d = 1; break; }
        dup[c] = d;
    }
    __syncthreads();

    // -- C. combine chunk statistics per row (one wave per row, lanes over chunks)
    for (int v = w; v < n1; v += kWalkWaves) {
        const float4* sv = stage ? sst + v * nchunk : stats + (seq + v) * nchunk;
        if (kGreedy) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            for (int c = lane; c < nchunk; c += kWave) {
                const float4 s4 = sv[c];
                argmax_merge(bv, bi, s4.x, __float_as_int(s4.y));
            }
            wave_argmax(bv, bi);
            if (lane == 0) info[v] = (bi >= 0 && bi < V) ? bi : 0;
        } else {
            const bool dr = info[v] != 0;
            float mt = -INFINITY, md = -INFINITY;
            for (int c = lane; c < nchunk; c += kWave) {
                const float4 s4 = sv[c];
                mt = fmaxf(mt, s4.x);
                if (dr) md = fmaxf(md, s4.z);
            }
            mt = wave_max(mt);
            md = wave_max(md);
            double st = 0.0, sd = 0.0;
            for (int c = lane; c < nchunk; c += kWave) {
                const float4 s4 = sv[c];
                if (s4.x != -INFINITY) st += static_cast<double>(s4.y) * __builtin_amdgcn_exp2f((s4.x - mt) * k);
                if (dr && s4.z != -INFINITY) sd += static_cast<double>(s4.w) * __builtin_amdgcn_exp2f((s4.z - md) * k);
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

    // -- D. per node: p, q of its token under its parent's rows, the ratio, its two uniforms
    for (int v = t; v < n1; v += kWalkThreads) {
        float pv = NAN, qv = NAN;
        if (!kGreedy) {
            const U64x4 rnd = philox4x64_10(static_cast<uint64_t>(v), static_cast<uint64_t>(b), offset, 0, seed, 0);
            uacc[v] = word_to_uniform(rnd.w[0]);
            ures[v] = word_to_uniform(rnd.w[1]);
            if (v > 0) {
                const int pa = par[v];
                const double zt = gzt, zd = gzd;
                const double lp = (zt - Mt[pa]) * invT;
                const double lq = (zd - Md[pa]) * invT;
                const double pd = exp(lp) / St[pa];
                const double qd = exp(lq) / Sd[pa];
                pq[v] = exp(lp - lq) * (Sd[pa] / St[pa]);
                qx[v] = static_cast<float>(qd);
                pv = static_cast<float>(pd);
                qv = static_cast<float>(qd);
            }
        }
        if (p_tok) p_tok[seq + v] = pv;
        if (q_tok) q_tok[seq + v] = qv;
    }
    __syncthreads();

    // -- E. the walk, run by wave 0; residual-mass passes (sibling rejections) use the whole block
    uint4 rt[kPassBatch], rd[kPassBatch];
    {
        int v = 0, n = 0;
        double cs = 0.0, R = 1.0, Q = 1.0, pend = 0.0;
        bool pending = false;
        int nxt = fch[0] < n1 ? fch[0] : -1;
        while (true) {
            if (w == 0) {
                if (pending) {
                    const double Rn = s_R;
                    if (Rn > 0.0) { cs = pend; R = Rn; }
                    pending = false;
                }
                int cmd = -1;   // 0: residual-mass pass, 1: draw at v, 2: greedy end at v
                while (cmd < 0) {
                    if (kGreedy) {
                        const int y = info[v];
                        int c = fch[v] < n1 ? fch[v] : -1;
                        while (c >= 0 && tok[c] != y) c = nsib[c];
                        if (c < 0) { cmd = 2; break; }
                        if (lane == 0) path[n] = c;
                        ++n;
                        v = c;
                        continue;
                    }
                    if (nxt < 0) { cmd = 1; break; }
                    const int c = nxt;
                    nxt = nsib[c];
                    if (dup[c]) continue;
                    const double ratio = fmax(0.0, pq[c] - cs) * Q / R;
                    if (uacc[c] < ratio) {
                        if (lane == 0) path[n] = c;
                        ++n;
                        v = c;
                        cs = 0.0; R = 1.0; Q = 1.0;
                        nxt = fch[v] < n1 ? fch[v] : -1;
                        continue;
                    }
                    const double cn = cs + R / Q;
                    Q -= static_cast<double>(qx[c]);
                    if (nxt >= 0) {
                        pending = true;
                        pend = cn;
                        if (lane == 0) {
                            s_ps = static_cast<float>(1.0 / St[v]);
                            s_qs = static_cast<float>(cn / Sd[v]);
                        }
                        cmd = 0;
                    } else {
                        cs = cn;
                        cmd = 1;
                    }
                }
                if (lane == 0) {
                    s_cmd = cmd;
                    s_row = v;
                    s_n = n;
                    if (cmd == 1) {
                        s_ps = static_cast<float>(1.0 / St[v]);
                        s_qs = (cs > 0.0) ? static_cast<float>(cs / Sd[v]) : 0.f;
                    }
                }
            }
            __syncthreads();
            if (s_cmd != 0) break;
            const int64_t rr = (seq + s_row) * V;
            const double Rn = row_pass<T, kVecOK>(target + rr, draft + rr, V, Mt[s_row], Md[s_row], k,
                                                  s_ps, s_qs, nullptr, red, rt, rd);
            if (t == 0) s_R = Rn;
            __syncthreads();
        }
    }

    // -- F. outputs of the walk
    const int cmd = s_cmd, e = s_row, na = s_n;
    for (int i = t; i < n1; i += kWalkThreads) {
        out_nodes[seq + i] = (i < na) ? path[i] : -1;
        if (i < na) out_tokens[seq + i] = tok[path[i]];
        else if (i > na) out_tokens[seq + i] = -1;
    }
    if (t == 0) accept_len[b] = na;
    if (cmd == 2) {
        if (t == 0) out_tokens[seq + na] = info[e];
        return;
    }

    // -- G. the draw at node e: w(x) = (p(x) - c q(x))+, smallest x whose CDF exceeds u * W
    const int64_t rr = (seq + e) * V;
    const float mt = Mt[e], ps = s_ps, qs = s_qs;
    const float md = (qs != 0.f) ? Md[e] : 0.f;
    const double W = row_pass<T, kVecOK>(target + rr, draft + rr, V, mt, md, k, ps, qs, seg, red, rt, rd);
    const int ntile = (V + kTile - 1) / kTile;
    const int nseg = ntile * kWalkWaves;
    const double thr = ures[e] * W;

    // -- H. wave 0 finds the segment holding the crossing (lane l owns a contiguous group)
    if (w == 0) {
        int sel = -1;
        double base = 0.0;
        if (W > 0.0) {
            const int g = (nseg + kWave - 1) / kWave;
            const int s0 = min(nseg, lane * g), s1 = min(nseg, s0 + g);
            double gs = 0.0;
            for (int i = s0; i < s1; ++i) gs += seg[i];
            double incl = gs;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const double yv = __shfl_up(incl, o);
                if (lane >= o) incl += yv;
            }
            const uint64_t hit = __ballot(s1 > s0 && incl > thr);
            int L;
            bool crossing;
            if (hit) {
                L = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                crossing = true;
            } else {   // rounding left u * W at or above every running sum: last group with mass
                const uint64_t nz = __ballot(gs > 0.0);
                L = nz ? 63 - __clzll(static_cast<long long>(nz)) : -1;
                crossing = false;
            }
            if (L >= 0 && lane == L) {
                double acc = incl - gs;
                int lastpos = -1;
                double lastbase = acc;
                for (int i = s0; i < s1; ++i) {
                    if (seg[i] > 0.f) { lastpos = i; lastbase = acc; }
                    if (crossing && acc + seg[i] > thr) { sel = i; base = acc; break; }
                    acc += seg[i];
                }
                if (sel < 0) { sel = lastpos; base = lastbase; }
            }
            if (L >= 0) {
                sel = __shfl(sel, L);
                base = __shfl(base, L);
            }
        }
        if (lane == 0) {
            s_sel = sel;
            s_base = base;
            s_found = -1;
        }
    }
    __syncthreads();

    // -- I. the wave owning the segment searches it, from registers when the whole row was held
    const int sel = s_sel;
    if (sel >= 0 && w == sel % kWalkWaves) {
        const int tile = sel / kWalkWaves;
        const int base = tile * kTile + (w * kWave + lane) * kVec;
        float zt[kVec], zd[kVec], wt[kVec];
        if (kVecOK && ntile <= kPassBatch) {
            uint4 a = rt[0], c = rd[0];
#pragma unroll
            for (int j = 1; j < kPassBatch; ++j)
                if (j == tile) { a = rt[j]; c = rd[j]; }
            if (base < V) {
                cvt_vec<T>(a, zt);
                cvt_vec<T>(c, zd);
            }
            if (!(base < V) || qs == 0.f) {
#pragma unroll
                for (int i = 0; i < kVec; ++i) {
                    zd[i] = -INFINITY;
                    if (!(base < V)) zt[i] = -INFINITY;
                }
            }
        } else {
            load_pair<T, kVecOK>(target + rr, draft + rr, V, base, qs != 0.f, zt, zd);
        }
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
            wt[i] = draw_weight(zt[i], zd[i], mt, md, k, ps, qs);
            ls += wt[i];
        }
        double incl2 = ls;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const double yv = __shfl_up(incl2, o);
            if (lane >= o) incl2 += yv;
        }
        double acc = s_base + incl2 - ls;
        int cand = INT_MAX, lastpos = -1;
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
            acc += wt[i];
            if (wt[i] > 0.f) {
                lastpos = base + i;
                if (cand == INT_MAX && acc > thr) cand = base + i;
            }
        }
        int y = -1;
        const uint64_t hit = __ballot(cand != INT_MAX);
        if (hit) {
            y = __shfl(cand, __ffsll(static_cast<unsigned long long>(hit)) - 1);
        } else {
            const uint64_t pos = __ballot(lastpos >= 0);
            if (pos) y = __shfl(lastpos, 63 - __clzll(static_cast<long long>(pos)));
        }
        if (lane == 0) s_found = y;
    }
    __syncthreads();
    int y = s_found;
    if (y < 0) {
        // no residual mass at all (a zero-probability event in exact arithmetic): the token with
        // the largest p(x) - c q(x), lowest index on ties
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int x = t; x < V; x += kWalkThreads) {
            const float zt = Elem<T>::load(target + rr, x);
            const float zd = (qs != 0.f) ? Elem<T>::load(draft + rr, x) : -INFINITY;
            const float d = __builtin_amdgcn_exp2f((zt - mt) * k) * ps - __builtin_amdgcn_exp2f((zd - md) * k) * qs;
            argmax_merge(bv, bi, d, x);
        }
        wave_argmax(bv, bi);
        __shared__ float pv[kWalkWaves];
        __shared__ int pi[kWalkWaves];
        if (lane == 0) { pv[w] = bv; pi[w] = bi; }
        __syncthreads();
        if (t == 0) {
            for (int i = 1; i < kWalkWaves; ++i) argmax_merge(pv[0], pi[0], pv[i], pi[i]);
            s_found = (pi[0] >= 0 && pi[0] < V) ? pi[0] : 0;
        }
        __syncthreads();
        y = s_found;
    }
    if (t == 0) out_tokens[seq + na] = y;
}

template <typename T, bool kVecOK>
hipError_t launch_typed(const AcceptArgs& a, hipStream_t stream) {
    constexpr int CH = chunk_elems<T>();
    const int nchunk = (a.V + CH - 1) / CH;
    const AcceptLayout lay(a.B, a.n1, nchunk);
    float4* stats = reinterpret_cast<float4*>(static_cast<char*>(a.workspace) + lay.stats);
    const T* target = static_cast<const T*>(a.target);
    const T* draft = static_cast<const T*>(a.draft);
    const bool greedy = a.temperature == 0.f;
    const double invT = greedy ? 0.0 : 1.0 / static_cast<double>(a.temperature);
    const float k = greedy ? 0.f : static_cast<float>(1.4426950408889634 * invT);   // log2(e) / T
    const dim3 sgrid(nchunk, a.n1, a.B);
    const bool all_draft = static_cast<double>(a.B) * a.n1 * a.V * sizeof(T) <= kAllDraftBytes;
    if (greedy) {
        hipLaunchKernelGGL((accept_stats_kernel<T, true, kVecOK, false>), sgrid, dim3(kStatThreads), 0, stream,
                           target, draft, a.parent, a.n1, a.V, nchunk, k, stats);
        hipLaunchKernelGGL((accept_finish_kernel<T, true, kVecOK>), dim3(a.B), dim3(kWalkThreads), 0, stream,
                           target, draft, a.tokens, a.parent, a.n1, a.V, nchunk, k, invT, a.seed, a.offset,
                           stats, a.accept_len, a.out_tokens, a.out_nodes, a.p_tok, a.q_tok);
    } else {
        if (all_draft)
            hipLaunchKernelGGL((accept_stats_kernel<T, false, kVecOK, true>), sgrid, dim3(kStatThreads), 0,
                               stream, target, draft, a.parent, a.n1, a.V, nchunk, k, stats);
        else
            hipLaunchKernelGGL((accept_stats_kernel<T, false, kVecOK, false>), sgrid, dim3(kStatThreads), 0,
                               stream, target, draft, a.parent, a.n1, a.V, nchunk, k, stats);
        hipLaunchKernelGGL((accept_finish_kernel<T, false, kVecOK>), dim3(a.B), dim3(kWalkThreads), 0, stream,
                           target, draft, a.tokens, a.parent, a.n1, a.V, nchunk, k, invT, a.seed, a.offset,
                           stats, a.accept_len, a.out_tokens, a.out_nodes, a.p_tok, a.q_tok);
    }
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
