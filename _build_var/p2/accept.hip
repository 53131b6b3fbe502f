// Exact accept / reject / resample over the vocabulary.
//
// [SD-EAGLE] "The Exactness Rule", [SD-review] §2: p = softmax(target / T), q = softmax(draft / T);
// accept x if u < p(x)/q(x); at the first rejection draw from (p - q)+ and stop; if the whole path
// is accepted draw a bonus token from p of the last node; greedy at T = 0.  [PTD] Method 4,
// "Acceptance Logic": on a tree the children of a node are tested in index order as draws without
// replacement from q; after i rejections the target is (p - c_i q)+ / R_i with c_0 = 0,
// R_0 = Q_0 = 1, c_{i+1} = c_i + R_i / Q_i (Q: draft mass not yet rejected).  Other sibling
// draftings take the same rule with their own proposal: i.i.d. draws keep q (Q stays 1, repeated
// tokens are tested); fixed candidates ([SD-EAGLE] "EAGLE: tree drafting and feature reuse",
// K candidates per depth) are point masses: x is accepted with probability p'(x) and dropped
// from p' when rejected, and the final draw excludes the rejected candidates.
//
// One launch whose grid never exceeds the number of workgroups the device holds at once (one per
// CU here: the LDS tables need about 100 KB).  Workgroups form teams of P; a team owns one
// sequence at a time (sequences are dealt to teams round-robin) and every phase that streams
// the vocabulary is split over the P workgroups of the team:
//   1. statistics: items (row, chunk of 64 * kVec * kWaveLoads elements), one wave per item, over
//      every target row and the draft rows of internal nodes, coalesced 16-byte loads, one exp per
//      element: per-chunk (R, sum of exp2(z k - R)) with k = log2e / T and the reference R the
//      chunk's largest z k (one fma per term), or (max, argmax) at T = 0.
//   2. every workgroup of the team combines the chunk statistics (fp64 above chunk level) and
//      builds per-node tables in LDS (p, q of each draft token under its parent's rows, p/q, both
//      Philox uniforms, first child / next sibling / repeated-token links);
//   3. one wave per workgroup runs the walk from those tables -- all workgroups of a team run the
//      same walk on the same data, so they take the same decisions;
//   4. residual-mass passes R(c) = sum (p - c q)+ (a rejection followed by another sibling) and the
//      final draw pass are split into P contiguous ranges; partial sums are exchanged and added in
//      rank order (fp64), so every workgroup sees the same totals.  The workgroup whose range holds
//      the CDF crossing searches it (per-segment sums in LDS, then one wave) and writes the token.
// Phase 1 can also run as a launch of its own just before (accept_stats_kernel: one wave per
// item over the whole device, the same item code, the same tagged words), after which the team
// kernel skips it.  That is the default where the team kernel would deal many items to each
// workgroup: dispatch then balances the stream across the device, which a static deal cannot.
// Workgroups exchange values through 64-bit words (32-bit value, 32-bit epoch of the launch)
// written and read with device-scope atomic stores / loads: a word carries its own validity, so
// no fence is needed.  The epoch lives in the workspace and advances by one per launch -- a replay
// of a captured launch included.
//
// No workgroup depends on another being scheduled.  A wait for a teammate's words (its chunk
// statistics, or its share of a vocabulary pass) lasts at most a budget (wait_ticks); after that
// the waiting workgroup computes the missing values itself, with the same arithmetic in the same
// order (a variant of the code that loads one vector at a time), so they are the same bits
// whoever computes them, and publishes them.  The outputs are therefore exact whatever the
// device does: a teammate that runs late (CUs held by another stream or process) costs time
// only.  Outputs are written by fixed workgroups (rank 0; the owner of the draw's CDF crossing),
// which all run eventually.
//
// Precision: per-element exponentials in fp32 (v_exp_f32) of z k - R rounded once (an fma),
// chunk and segment sums in fp32, everything above (row normalisers, ratios, c, Q, R, the CDF
// threshold and prefixes) in fp64; team partial sums cross workgroups as fp64 (two words).  A
// reference is kept at or above -FLT_MAX, so a row whose logits all lie below -FLT_MAX / k (about
// -2.4e38 T), like a row of -inf, has no probability mass.

#include <algorithm>
#include <cfloat>
#include <atomic>
#include <cstdlib>

#include "common.h"
#include "kernels.h"

// No contraction of multiplies and adds into fma in this file: a value that one workgroup
// computes on behalf of another must be the same bits as the owner's, and with contraction the
// choice could differ between two inlined copies of the same code.  (The fmas that the code
// writes out, __builtin_fmaf, are the same operation in every copy.)
#pragma clang fp contract(off)

namespace specv {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kWaveLoads = 16;              // 16-byte loads per lane per statistics item
constexpr int kMaxVocab = 1 << 21;
constexpr int kMaxTeam = 64;                // workgroups per sequence at most
constexpr int kPassBatch = 4;               // tiles per batch of a range pass
constexpr int kBufferWord3 = 0x00020000;    // raw buffer descriptor, word 3 (CDNA)
// how the siblings of a node were drafted (the walk is the recursive rejection rule with the
// proposal each sibling was drawn from)
constexpr int kRuleWithoutReplacement = 0;  // drawn without replacement from q_v
constexpr int kRuleIid = 1;                 // drawn independently from q_v
constexpr int kRuleDeterministic = 2;       // fixed candidates (a point mass each)
constexpr int kMaskNodes = 128;             // trees up to this size keep children bit masks
constexpr int kMaskWords = kMaskNodes / 64;
constexpr int kLine = 8;                    // 64-bit words per control line (64 bytes)

template <typename T>
constexpr int item_elems() { return kWave * Elem<T>::kVec * kWaveLoads; }   // bf16 8192, fp32 4096

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ctl: the epoch (word 0), counts of batches of statistics (word 1) and of range partials (word 2)
// computed on a teammate's behalf since the workspace was cleared (diagnostics); seen: the epoch
// each workgroup last held [B * P] (32 bits); stat: tagged chunk statistics [B][n1][nchunk][4];
// part: tagged fp64 partial sums of the team exchanges [B][n1 + 1][P][2].
struct AcceptLayout {
    size_t ctl, seen, stat, part, total;
    AcceptLayout(int B, int n1, int nchunk, int P) {
        ctl = 0;
        seen = align256(ctl + sizeof(uint64_t) * kLine);
        stat = align256(seen + sizeof(uint32_t) * size_t(B) * P);
        part = align256(stat + sizeof(uint64_t) * size_t(B) * n1 * nchunk * 4);
        total = align256(part + sizeof(uint64_t) * size_t(B) * (n1 + 1) * P * 2);
    }
};

// ---------------------------------------------------------------------------------- helpers

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

// Draw weight of one element: (p(x) - c q(x))+ with p = exp2(zt k - rt) / S_t (rt the row's
// reference), q likewise.
__device__ __forceinline__ float draw_weight(float zt, float zd, float rt, float rd, float k,
                                             float p_scale, float q_scale) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(zt, k, -rt)) * p_scale;
    const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(zd, k, -rd)) * q_scale;
    return fmaxf(p - q, 0.0f);
}

// The 16-byte words of one statistics item: lane l gets vectors u * 64 + l (u < kWaveLoads) of
// the element range [lo, hi) of `row`.  Buffer loads: one descriptor per wave (row, lo and hi are
// wave-uniform) and one offset register for all loads, the vector index in the immediate part,
// so nothing per load stays live; vectors past hi come back as 0 from the range check (whole
// vectors: V is a multiple of the vector length on this path) and are masked where used.
template <typename T>
__device__ __forceinline__ void load_item(const T* row, int lo, int hi, int lane, uint4 (&r)[kWaveLoads]) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(row + lo), 0, (hi - lo) * static_cast<int>(sizeof(T)), kBufferWord3);
#pragma unroll
    for (int u = 0; u < kWaveLoads; ++u) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, u * kWave * 16, kCachePolicyNT);
        r[u] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// A logit's raw bits in a 32-bit word, and back as fp32 (bf16: its bits in the high half; exact).
__device__ __forceinline__ uint32_t raw_bits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t raw_bits(uint16_t x) { return x; }
template <typename T>
__device__ __forceinline__ float widen(uint32_t b) { return __uint_as_float(sizeof(T) == 2 ? b << 16 : b); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations (and scalar
// loads), not for its global loads still in flight, which __syncthreads would also wait for.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Publish a tagged 64-bit word (value in the low half, the launch's epoch in the high half).
__device__ __forceinline__ void put_word(uint64_t* p, uint32_t bits, uint32_t tag) {
    __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | bits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_word(uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// An fp64 value as two tagged words (high half first).
__device__ __forceinline__ void put_double(uint64_t* p, double x, uint32_t tag) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x));
    put_word(p, static_cast<uint32_t>(b >> 32), tag);
    put_word(p + 1, static_cast<uint32_t>(b), tag);
}

// Wait at most `budget` ticks of the 100 MHz wall clock for both words of an fp64 value (both
// requested together, then whichever is missing polled); true if they came, with the value.
__device__ bool get_double(uint64_t* p, uint32_t tag, uint64_t budget, double* out) {
    uint64_t w0 = load_word(p), w1 = load_word(p + 1);
    auto absent = [&]() {
        return static_cast<uint32_t>(w0 >> 32) != tag || static_cast<uint32_t>(w1 >> 32) != tag;
    };
    if (absent()) {
        const uint64_t t0 = wall_clock64();
        do {
            if (wall_clock64() - t0 > budget) return false;
            __builtin_amdgcn_s_sleep(1);
            if (static_cast<uint32_t>(w0 >> 32) != tag) w0 = load_word(p);
            if (static_cast<uint32_t>(w1 >> 32) != tag) w1 = load_word(p + 1);
        } while (absent());
    }
    *out = __longlong_as_double(static_cast<long long>((w0 << 32) | (w1 & 0xFFFFFFFFull)));
    return true;
}

// Bit e set iff token base + e is in the exclusion list (tokens whose weight is 0 in a draw:
// the rejected candidates under the deterministic sibling rule; the list is short).
__device__ __forceinline__ uint32_t excluded_in(const int32_t* excl, int nexcl, int base) {
    uint32_t m = 0;
    for (int j = 0; j < nexcl; ++j) {
        const uint32_t d = static_cast<uint32_t>(excl[j] - base);
        m |= (d < 32u) ? (1u << d) : 0u;
    }
    return m;
}

// The statistics of one item (one wave): (R, sum of exp2(z k - R)) over elements [lo, hi) of
// `src`, R the largest z k (kept at or above -FLT_MAX), or (max, argmax) at T = 0, as two words
// (w0, w1; in every lane).  The wave's lanes
// take the item's 16-byte vectors u = 0 .. kWaveLoads - 1 in order; `r` holds their raw words if
// `loaded`, else they are loaded here, all at once -- or, with kLean, one at a time (few
// registers, same arithmetic in the same order, so the same bits).
template <typename T, bool kGreedy, bool kVecOK, bool kLean>
__device__ __forceinline__ void item_stats(const T* src, int lo, int hi, int lane, float k, uint4 (&r)[kWaveLoads],
                                           bool loaded, uint32_t& w0, uint32_t& w1) {
    constexpr int kVec = Elem<T>::kVec;
    if (kVecOK && !kLean && !loaded) load_item<T>(src, lo, hi, lane, r);
    // values of vector u, converted from the raw words when used (two passes: max, then sum of
    // exp), so only the raw 16-byte words stay in registers
    auto values = [&](int u, float* z) {
        const int base = lo + (u * kWave + lane) * kVec;
        if (kVecOK) {
            uint4 rv;
            if constexpr (kLean) {
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<T*>(src + lo), 0, (hi - lo) * static_cast<int>(sizeof(T)), kBufferWord3);
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, u * kWave * 16, kCachePolicyNT);
                rv = make_uint4(v[0], v[1], v[2], v[3]);
            } else {
                rv = r[u];
            }
            // (a vector lies wholly inside or outside the row: outside, its raw words become
            // -inf; selects, no branches)
            const bool in = base < hi;
            constexpr uint32_t kNegInf = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;
            rv.x = in ? rv.x : kNegInf;
            rv.y = in ? rv.y : kNegInf;
            rv.z = in ? rv.z : kNegInf;
            rv.w = in ? rv.w : kNegInf;
            cvt_vec<T>(rv, z);
        } else {
#pragma unroll
            for (int e = 0; e < kVec; ++e) z[e] = (base + e < hi) ? Elem<T>::load(src, base + e) : -INFINITY;
        }
    };
    if (kGreedy) {
        // this lane's elements come in increasing index order, so a strict > keeps the lowest
        // index among equal values; branch-free selects; kVec independent running maxima (one
        // per vector position), merged at the end
        float bv = -INFINITY;
        int bi = INT_MAX;
        float bvs[kVec];
        int bis[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) { bvs[e] = -INFINITY; bis[e] = INT_MAX; }
        auto scan = [&](int u) {
            float z[kVec];
            values(u, z);
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const int x = lo + (u * kWave + lane) * kVec + e;
                const bool take = (z[e] > bvs[e]) & (x < hi);
                bvs[e] = take ? z[e] : bvs[e];
                bis[e] = take ? x : bis[e];
            }
        };
        if constexpr (kVecOK && !kLean) {
#pragma unroll
            for (int u = 0; u < kWaveLoads; ++u) scan(u);
        } else {
#pragma nounroll
            for (int u = 0; u < kWaveLoads; ++u) scan(u);
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) argmax_merge(bv, bi, bvs[e], bis[e]);
        wave_argmax(bv, bi);
        w0 = __float_as_uint(bv);
        w1 = static_cast<uint32_t>(bi);
    } else {
        // online over the 16-byte vectors in the scaled domain: the reference R is the largest
        // z k so far, each term exp2(z k - R) with the argument rounded once (an fma), and the
        // running sum is rescaled once per vector.  R starts at, and never goes below, -FLT_MAX,
        // so no term or rescale factor is ever NaN (terms of -inf logits are 0) and no branch or
        // select guards it.
        float R = -FLT_MAX, sum = 0.f;
        auto fold = [&](int u) {
            float z[kVec];
            values(u, z);
            float mu = -INFINITY;
#pragma unroll
            for (int e = 0; e < kVec; ++e) mu = fmaxf(mu, z[e]);
            const float Ru = fmaxf(R, fmaxf(mu * k, -FLT_MAX));
            float add = 0.f;
#pragma unroll
            for (int e = 0; e < kVec; ++e) add += __builtin_amdgcn_exp2f(__builtin_fmaf(z[e], k, -Ru));
            sum = __builtin_fmaf(sum, __builtin_amdgcn_exp2f(R - Ru), add);
            R = Ru;
        };
        if constexpr (kVecOK && !kLean) {
#pragma unroll
            for (int u = 0; u < kWaveLoads; ++u) fold(u);
        } else {
#pragma nounroll
            for (int u = 0; u < kWaveLoads; ++u) fold(u);
        }
        wave_max_sum(R, sum, 1.0f);      // (references already scaled)
        w0 = __float_as_uint(R);
        w1 = __float_as_uint(sum);
    }
}

// Streaming pass over tiles [t0, t1) of one row pair with the draw weights.  Tile i covers
// kThreads * kVec consecutive elements; within a tile wave ww owns the contiguous segment of
// 64 * kVec elements at (ww * 64) * kVec.  Segment sums go to seg[(i - t0) * kWaves + ww] if seg is
// given.  Up to kBatch tiles are loaded together; the raw words of the last batch stay in rt /
// rd.  Returns the block's total (fp64, identical in all threads).
template <typename T, bool kVecOK, int kBatch = kPassBatch>
__device__ __forceinline__ double range_pass(const T* __restrict__ trow, const T* __restrict__ drow, int V, int t0,
                             int t1, float mt, float md, float k, float p_scale, float q_scale,
                             const int32_t* excl, int nexcl,
                             float* seg, double* red, uint4 (&rt)[kBatch], uint4 (&rd)[kBatch]) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int kTile = kThreads * kVec;
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const bool use_q = q_scale != 0.f;
    double acc = 0.0;
    for (int i0 = t0; i0 < t1; i0 += kBatch) {
        if (kVecOK) {
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int base = (i0 + j) * kTile + threadIdx.x * kVec;
                rt[j] = make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
                rd[j] = rt[j];
                if (i0 + j < t1 && base < V) {
                    rt[j] = load_nt(trow + base);
                    if (use_q) rd[j] = load_nt(drow + base);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (i0 + j >= t1) break;
            const int base = (i0 + j) * kTile + threadIdx.x * kVec;
            float zt[kVec], zd[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) { zt[e] = -INFINITY; zd[e] = -INFINITY; }
            if (kVecOK) {
                if (base < V) {
                    cvt_vec<T>(rt[j], zt);
                    if (use_q) cvt_vec<T>(rd[j], zd);
                }
            } else {
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    if (base + e < V) {
                        zt[e] = Elem<T>::load(trow, base + e);
                        if (use_q) zd[e] = Elem<T>::load(drow, base + e);
                    }
                }
            }
            const uint32_t xm = excluded_in(excl, nexcl, base);
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < kVec; ++e)
                sum += ((xm >> e) & 1u) ? 0.f : draw_weight(zt[e], zd[e], mt, md, k, p_scale, q_scale);
            sum = wave_sum(sum);
            if (seg && lane == 0) seg[(i0 + j - t0) * kWaves + w] = sum;
            acc += sum;
        }
    }
    __syncthreads();
    if (lane == 0) red[w] = acc;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) tot += red[i];
    __syncthreads();
    return tot;
}

// The same pass, one tile at a time (few registers; the same sums in the same order, so the same
// bits): computes a teammate's share when it runs late.
template <typename T, bool kVecOK>
__device__ __forceinline__ double range_pass_lean(const T* trow, const T* drow, int V, int t0, int t1, float mt,
                                                  float md, float k, float p_scale, float q_scale,
                                                  const int32_t* excl, int nexcl, double* red) {
    uint4 xt[1], xd[1];
    return range_pass<T, kVecOK, 1>(trow, drow, V, t0, t1, mt, md, k, p_scale, q_scale, excl, nexcl, nullptr, red,
                                    xt, xd);
}

// Team exchange of fp64 partial sums (two tagged words each).  exchange_post publishes this
// workgroup's partial, reads the team's P partials into s_vals, waiting at most `budget` for
// each, and returns the mask of those still missing then (the same in every thread; P <= 64, so
// wave 0 does the reads).  The caller computes each missing partial itself and hands it to
// exchange_fill; exchange_sum adds them in rank order, so every workgroup of the team gets the
// same prefix and total.
__device__ __forceinline__ uint64_t exchange_post(uint64_t* slots, int P, int rank, double mine, uint32_t tag,
                                                  uint64_t budget, double* s_vals, uint64_t* s_mask) {
    const int t = threadIdx.x;
    if (t == 0) put_double(slots + 2 * rank, mine, tag);
    if (t < kWave) {
        bool miss = false;
        if (t < P) {
            double v = mine;
            if (t != rank && !get_double(slots + 2 * t, tag, budget, &v)) miss = true;
            s_vals[t] = v;
        }
        const uint64_t m = __ballot(miss);
        if (t == 0) *s_mask = m;
    }
    __syncthreads();
    return *s_mask;
}

// Every thread stores the value (the same in all; each reads its own store afterwards); thread 0
// publishes it for the other workgroups and counts it at *counter.
__device__ __forceinline__ void exchange_fill(uint64_t* slots, int r, double v, uint32_t tag, double* s_vals,
                                              uint64_t* counter) {
    s_vals[r] = v;
    if (threadIdx.x == 0) {
        put_double(slots + 2 * r, v, tag);
        __hip_atomic_fetch_add(counter, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ void exchange_sum(const double* s_vals, int P, int rank, double& before, double& total) {
    before = 0.0;
    total = 0.0;
    for (int r = 0; r < P; ++r) {
        if (r < rank) before += s_vals[r];
        total += s_vals[r];
    }
}

// ---------------------------------------------------------------------------------- statistics launch

constexpr int kStatThreads = 256;               // 4 waves, one item each
constexpr int kStatWaves = kStatThreads / kWave;

// The launch's tag: the workspace epoch + 1 (0 is the tag of a zero-filled word; the epoch
// 0xFFFFFFFF wraps to tag 1).
__device__ __forceinline__ uint32_t tag_of(uint32_t epoch) { return epoch == 0xFFFFFFFFu ? 1u : epoch + 1u; }

// Phase 1 as a launch of its own: one wave per item (row, chunk) of every sequence -- all target
// rows, then the draft rows of internal nodes -- writing the tagged chunk statistics the team
// kernel reads, with the same arithmetic (item_stats, same template), so the same bits.  The
// workgroups are independent and short, so the device's dispatcher spreads the vocabulary stream
// over every compute unit as they free up: no static deal, no teammate to wait for.  A draft
// item first checks that its row has a child (any parent[b][c] == row); a leaf's draft row is not
// read.  The tag is the one the team kernel that follows on the stream will use: it reads the
// same epoch, which only that kernel advances.
template <typename T, bool kGreedy, bool kVecOK>
__global__ void __launch_bounds__(kStatThreads)
accept_stats_kernel(const T* __restrict__ target, const T* __restrict__ draft, const int32_t* __restrict__ parent,
                    int B, int n1, int V, int nchunk, int with_draft, float k, const uint64_t* __restrict__ ctl,
                    uint64_t* __restrict__ statw) {
    constexpr int kItem = item_elems<T>();
    const int lane = threadIdx.x % kWave;
    const int wu = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    const int64_t tgt_items = static_cast<int64_t>(n1) * nchunk;
    const int64_t per_seq = tgt_items * (with_draft ? 2 : 1);
    const int64_t total = per_seq * B;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kStatWaves;
    const uint32_t tag = tag_of(static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(load_word(const_cast<uint64_t*>(ctl))))));
    for (int64_t it = static_cast<int64_t>(blockIdx.x) * kStatWaves + wu; it < total; it += stride) {
        const int64_t b = it / per_seq, j0 = it - b * per_seq;
        const bool isd = j0 >= tgt_items;
        const int64_t j = isd ? j0 - tgt_items : j0;
        const int row = static_cast<int>(j / nchunk), c = static_cast<int>(j - static_cast<int64_t>(row) * nchunk);
        const int64_t seq = b * n1;
        if (isd) {
            // only rows with a child are read (values of parent are compared, never used as indices)
            bool f = false;
            for (int i = 1 + lane; i < n1; i += kWave) f |= parent[seq + i] == row;
            if (__ballot(f) == 0) continue;      // (wave-uniform)
        }
        const T* src = (isd ? draft : target) + (seq + row) * V;
        const int lo = c * kItem, hi = min(V, lo + kItem);
        uint4 r[kWaveLoads];
        uint32_t w0, w1;
        item_stats<T, kGreedy, kVecOK, false>(src, lo, hi, lane, k, r, false, w0, w1);
        if (lane == 0) {
            uint64_t* slot = statw + ((seq + row) * nchunk + c) * 4 + (isd ? 2 : 0);
            put_word(slot, w0, tag);
            put_word(slot + 1, w1, tag);
        }
    }
}

// ---------------------------------------------------------------------------------- the kernel

template <typename T, bool kGreedy, bool kVecOK>
__global__ void __launch_bounds__(kThreads)
accept_kernel(const T* __restrict__ target, const T* __restrict__ draft,
              const int32_t* __restrict__ tokens, const int32_t* __restrict__ parent, int B, int n1,
              int V, int nchunk, int P, int rule, float k, uint64_t seed, uint64_t offset, int stats_ready,
              uint64_t* __restrict__ ctl, uint32_t* __restrict__ seen, uint64_t wait_ticks,
              uint64_t* __restrict__ statw, uint64_t* __restrict__ partw, int32_t* __restrict__ accept_len,
              int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_nodes,
              float* __restrict__ p_tok, float* __restrict__ q_tok) {
    constexpr int kVec = Elem<T>::kVec;
    constexpr int kTile = kThreads * kVec;
    constexpr int kItem = item_elems<T>();
    constexpr int kMaxSeg = (kMaxVocab + kTile - 1) / kTile * kWaves;
    // first statistics item loaded during A and B: bf16 logits only (with fp32 logits the longer
    // live ranges make the compiler spill there, and waiting on the spill reloads would wait on
    // the item anyway)
    constexpr bool kPre = kVecOK && sizeof(T) == 2;
    __shared__ int32_t par[kMaxNodes];
    __shared__ int32_t tok[kMaxNodes];
    __shared__ int32_t info[kMaxNodes];     // greedy: argmax token of the row; else: has children
    __shared__ int32_t fch[kMaxNodes];      // first child (n1 if none)
    __shared__ int32_t nsib[kMaxNodes];     // next sibling (-1 if none)
    __shared__ int32_t dup[kMaxNodes];      // token repeats an earlier sibling's
    __shared__ uint64_t cmask[kMaskNodes][kMaskWords];   // children of each node as a bit mask
    __shared__ int32_t ilist[kMaxNodes];    // internal rows in index order
    __shared__ float Mt[kMaxNodes], Md[kMaxNodes];   // row references (largest z k; scaled domain)
    __shared__ double St[kMaxNodes], Sd[kMaxNodes];
    __shared__ double pq[kMaxNodes];        // p(x)/q(x) of node x under its parent's rows
    __shared__ float qx[kMaxNodes];         // q(x)
    __shared__ double uacc[kMaxNodes];      // acceptance uniforms
    __shared__ double ures[kMaxNodes];      // draw uniforms
    __shared__ int32_t path[kMaxNodes];
    __shared__ float seg[kMaxSeg];
    __shared__ double red[kWaves];
    __shared__ double s_vals[kMaxTeam];
    __shared__ int wcount[kWaves];
    __shared__ float pv[kWaves];
    __shared__ int pi[kWaves];
    __shared__ int s_bad, s_ni, s_cmd, s_row, s_n, s_sel, s_found, s_late, s_next, s_nexcl;
    __shared__ uint64_t s_mask;
    __shared__ float s_ps, s_qs;
    __shared__ double s_R, s_base;

    const int t = threadIdx.x;
    const int w = t / kWave, lane = t % kWave;
    const int wu = __builtin_amdgcn_readfirstlane(w);      // the same, known wave-uniform
    const int team = blockIdx.x / P, rank = blockIdx.x % P, nteams = gridDim.x / P;
    const int ntile = (V + kTile - 1) / kTile;
    const int tpb = (ntile + P - 1) / P;
    const int my_t0 = min(ntile, rank * tpb), my_t1 = min(ntile, my_t0 + tpb);

    // This launch's epoch: ctl[0] + 1 (0 is the tag of a zero-filled word), loaded in A of the
    // workgroup's first sequence beside the parent array (so nothing waits for it alone).  Once
    // a workgroup holds it, it stores it in its slot of `seen` (after the load has returned, so
    // that no later read can see a newer epoch); workgroup 0 advances the epoch when it leaves,
    // after it has seen every slot hold it.  (Plain stores, no contended counter; workgroup 0 is
    // rarely the last to finish.)
    uint32_t tag = 0, epoch_raw = 0;
    if (t == 0) s_late = 0;     // (ordered by the barriers of A)
    for (int b = team; b < B; b += nteams) {
        const int64_t seq = static_cast<int64_t>(b) * n1;
        uint64_t* sw = statw + seq * nchunk * 4;
        uint64_t* pw = partw + static_cast<int64_t>(b) * (n1 + 1) * P * 2;

        // -- A. stage and validate the parent array and the draft tokens.  The barriers of A and
        //    B order LDS only, so the loads of this wave's first statistics item, issued here when
        //    it is a target-row chunk (those do not depend on the tree), stay in flight through A
        //    and B.  Every thread first loads one parent and token (clamped index), so that waiting
        //    for them does not mean waiting for the item.
        lds_barrier();
        if (t == 0) {
            s_bad = 0;
            s_next = kWaves;      // the first kWaves takes of the statistics phase are by position
        }
        for (int i = t; i < n1; i += kThreads) {
            info[i] = 0;
            fch[i] = n1;
        }
        for (int i = t; i < kMaskNodes * kMaskWords; i += kThreads) cmask[i / kMaskWords][i % kMaskWords] = 0;
        // (relaxed atomic loads: unlike loads of read-only arguments the compiler does not sink
        // them below the barrier, so they are issued ahead of the item's loads)
        const bool first_seq = b == team;
        if (first_seq)
            epoch_raw = static_cast<uint32_t>(__hip_atomic_load(ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        const int pa0 = __hip_atomic_load(parent + seq + min(t, n1 - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int xa0 = __hip_atomic_load(tokens + seq + min(t, n1 - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        asm volatile("" ::: "memory");
        uint4 r[kWaveLoads];
        const int it0 = rank + wu * P;
        const bool pre = kPre && !stats_ready && it0 < n1 * nchunk;       // wave-uniform
        if constexpr (kPre) {
            // issued by every wave (branch-free, so the compiler's count of outstanding loads
            // stays exact); a wave without a target-row first item gets an empty range, whose
            // loads return without touching memory
            const int i0 = min(it0, n1 * nchunk - 1), lo = (i0 % nchunk) * kItem;
            load_item<T>(target + (seq + i0 / nchunk) * V, lo, pre ? min(V, lo + kItem) : lo, lane, r);
        }
        lds_barrier();
        for (int i = t; i < n1; i += kThreads) {
            const int p = i == t ? pa0 : parent[seq + i];
            const int x = i == t ? xa0 : tokens[seq + i];
            par[i] = p;
            tok[i] = x;
            const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i && x >= 0 && x < V);
            if (!ok) s_bad = 1;
        }
        if (first_seq) {
            tag = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(tag_of(epoch_raw))));
            if (t == 0) __hip_atomic_store(seen + blockIdx.x, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        lds_barrier();
        if (s_bad) {
            if (rank == 0) {
                for (int i = t; i < n1; i += kThreads) {
                    out_tokens[seq + i] = -1;
                    out_nodes[seq + i] = -1;
                    if (p_tok) p_tok[seq + i] = NAN;
                    if (q_tok) q_tok[seq + i] = NAN;
                }
                if (t == 0) accept_len[b] = -1;
            }
            continue;
        }

        // -- B. tree links, internal rows; gather every draft token's logits under its parent's rows
        // (raw bits, made opaque and widened only in E, so that nothing waits for them before)
        uint32_t gzt = 0, gzd = 0;
        if (!kGreedy && t > 0 && t < n1) {
            const int pa = par[t], x = tok[t];
            const int64_t gi = (seq + SPECV_CHK(pa, n1, kSiteAcceptGatherRow)) * V + SPECV_CHK(x, V, kSiteAcceptGatherToken);
            gzt = raw_bits(target[gi]);
            if (rule != kRuleDeterministic) gzd = raw_bits(draft[gi]);
        }
        // both uniforms of every node (Philox; computed while the gathers are in flight)
        if (!kGreedy) {
            for (int v = t; v < n1; v += kThreads) {
                const U64x4 rnd = philox4x64_10(static_cast<uint64_t>(v), static_cast<uint64_t>(b), offset, 0, seed, 0);
                uacc[v] = word_to_uniform(rnd.w[0]);
                ures[v] = word_to_uniform(rnd.w[1]);
            }
        }
        // first child of every parent; for trees of at most kMaskNodes nodes also each parent's
        // children as a bit mask, from which next siblings and repeated tokens follow after the
        // barrier
        const bool small = n1 <= kMaskNodes;
        for (int c = 1 + t; c < n1; c += kThreads) {
            const int pa = par[c];
            info[SPECV_CHK(pa, n1, kSiteAcceptLink)] = 1;
            atomicMin(&fch[SPECV_CHK(pa, n1, kSiteAcceptLink)], c);
            if (small) atomicOr(&cmask[SPECV_CHK(pa, kMaskNodes, kSiteAcceptLink)][c >> 6], 1ull << (c & 63));
        }
        if (!small) {
            // larger trees: each wave walks all nodes 64 at a time, one LDS read per lane, the
            // values handed to every lane by readlane; next sibling = smallest i > c with the same
            // parent, repeated token = an earlier sibling with the same token
            for (int c0 = 1 + wu * kWave; c0 < n1; c0 += kThreads) {     // wave-uniform
                const int c = c0 + lane;
                const bool valid = c < n1;
                const int pa = valid ? par[c] : -3;
                const int x = valid ? tok[c] : -1;
                int nx = INT_MAX, d = 0;
                for (int base = 0; base < n1; base += kWave) {
                    const int i0 = base + lane;
                    const int pl = i0 < n1 ? par[i0] : -2;
                    const int tl = i0 < n1 ? tok[i0] : -1;
                    const int cnt = min(kWave, n1 - base);
                    for (int j = 0; j < cnt; ++j) {
                        const int pi = __builtin_amdgcn_readlane(pl, j);
                        const int ti = __builtin_amdgcn_readlane(tl, j);
                        const int i = base + j;
                        const bool same = pi == pa;
                        nx = (same && i > c) ? min(nx, i) : nx;
                        d |= (same && i < c && ti == x) ? 1 : 0;
                    }
                }
                if (valid) {
                    nsib[c] = nx == INT_MAX ? -1 : nx;
                    dup[c] = d;
                }
            }
        }
        lds_barrier();
        if (small) {
            for (int c = 1 + t; c < n1; c += kThreads) {
                const int x = tok[c], pa = par[c], cw = c >> 6, cb = c & 63;
                int nx = -1, d = 0;
#pragma unroll
                for (int q = kMaskWords - 1; q >= 0; --q) {
                    const uint64_t m = cmask[SPECV_CHK(pa, kMaskNodes, kSiteAcceptLink)][q];
                    // siblings after c in this word (all of it if the word is past c's; cb <= 63,
                    // so 2 << cb wraps to 0 only for cb == 63, leaving no bits)
                    const uint64_t later = q > cw ? m : (q == cw ? m & ~((2ull << cb) - 1ull) : 0ull);
                    if (later) nx = 64 * q + __builtin_ctzll(later);
                    uint64_t earlier = q < cw ? m : (q == cw ? m & ((1ull << cb) - 1ull) : 0ull);
                    while (earlier) {
                        d |= tok[64 * q + __builtin_ctzll(earlier)] == x;
                        earlier &= earlier - 1ull;
                    }
                }
                nsib[c] = nx;
                dup[c] = d;
            }
        }
        {   // compact list of internal rows, in index order
            int done = 0;
            for (int base = 0; base < n1; base += kThreads) {
                const int v = base + t;
                const bool f = v < n1 && info[v] != 0;
                const uint64_t m = __ballot(f);
                if (lane == 0) wcount[w] = __popcll(m);
                lds_barrier();
                int before = 0, all = 0;
                for (int i = 0; i < kWaves; ++i) {
                    if (i < w) before += wcount[i];
                    all += wcount[i];
                }
                if (f) ilist[done + before + __popcll(m & ((1ull << lane) - 1ull))] = v;
                done += all;
                lds_barrier();
            }
            if (t == 0) s_ni = done;
            lds_barrier();
        }
        const int ni = (kGreedy || rule == kRuleDeterministic) ? 0 : s_ni;     // draft rows read

        // -- C. chunk statistics: one wave per item.  Workgroup `rank` of the team owns items
        //    rank + m * P (dealt one at a time, so the workgroups' counts differ by at most one);
        //    its waves take them in that order from a workgroup counter in LDS as they finish,
        //    since the two waves sharing a SIMD do not progress at the same rate (the older one is
        //    favoured at issue), which a fixed split would turn into idle waves at the end of the
        //    phase
        //    (nothing to do here when the statistics launch has written them)
        const int nitems = stats_ready ? 0 : (n1 + ni) * nchunk;
        for (int kk = wu;;) {     // (wave-uniform)
            const int it = rank + kk * P;
            if (it >= nitems) break;
            int nk = 0;
            if (lane == 0) nk = atomicAdd(&s_next, 1);
            nk = __builtin_amdgcn_readfirstlane(nk);
            const bool isd = it >= n1 * nchunk;
            const int j = isd ? it - n1 * nchunk : it;
            const int row = isd ? __builtin_amdgcn_readfirstlane(ilist[j / nchunk]) : j / nchunk;
            const int c = j % nchunk;
            const T* src = (isd ? draft : target) + (seq + row) * V;
            const int lo = c * kItem, hi = min(V, lo + kItem);
            uint64_t* slot = sw + (static_cast<int64_t>(row) * nchunk + c) * 4 + (isd ? 2 : 0);
            // (the wave's first item, kk == w, was loaded in A when `pre`)
            uint32_t w0, w1;
            item_stats<T, kGreedy, kVecOK, false>(src, lo, hi, lane, k, r, pre && kk == wu, w0, w1);
            if (lane == 0) {
                put_word(slot, w0, tag);
                put_word(slot + 1, w1, tag);
            }
            kk = nk;
        }

        // -- D. combine the chunk statistics of every row.  Rows go in batches whose words fit the
        //    segment buffer (free until the draw): each thread reads its share of the batch's
        //    tagged words into LDS -- every load issued first, the words not yet published then
        //    polled together -- so the whole batch costs about one round trip; then g lanes per row
        //    (g = chunk count rounded up to a power of two, at most 64) reduce them, fp64 above
        //    chunk level.  (A row has at most 256 bf16 / 512 fp32 chunks, 4 words each, so one row
        //    always fits.)
        {
            constexpr int kStage = kMaxSeg / kThreads;
            const int rw = nchunk * 4;
            const int rb = min(n1, kMaxSeg / rw);
            int g = 1;
            while (g < nchunk && g < kWave) g <<= 1;
            const int rpw = kWave / g, sub = lane / g, cl = lane % g;
            for (int r0 = 0; r0 < n1; r0 += rb) {
                const int nr = min(rb, n1 - r0);
                const int nw = nr * rw;
                uint64_t* src = sw + static_cast<int64_t>(r0) * rw;
                uint64_t raw[kStage];
                bool need[kStage];
#pragma unroll
                for (int j = 0; j < kStage; ++j) {
                    const int i = t + j * kThreads;
                    const int wi = i & 3;
                    need[j] = i < nw && (wi < 2 || (!kGreedy && rule != kRuleDeterministic && info[r0 + i / rw] != 0));
                    raw[j] = need[j] ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
                }
                auto missing = [&]() {
                    bool any = false;
#pragma unroll
                    for (int j = 0; j < kStage; ++j) any |= need[j] && static_cast<uint32_t>(raw[j] >> 32) != tag;
                    return any;
                };
                if (missing()) {
                    const uint64_t t0 = wall_clock64();
                    do {
                        __builtin_amdgcn_s_sleep(1);
#pragma unroll
                        for (int j = 0; j < kStage; ++j)
                            if (need[j] && static_cast<uint32_t>(raw[j] >> 32) != tag)
                                raw[j] = __hip_atomic_load(src + t + j * kThreads, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                        if (wall_clock64() - t0 > wait_ticks) {
                            s_late = 1;
                            break;
                        }
                    } while (missing());
                }
#pragma unroll
                for (int j = 0; j < kStage; ++j)
                    if (need[j]) seg[t + j * kThreads] = __uint_as_float(static_cast<uint32_t>(raw[j]));
                __syncthreads();
                if (s_late) {
                    // rare: words of the batch still missing after the wait.  Each wave checks 64
                    // of the batch's items at a time (item q: words 2q, 2q + 1) and computes the
                    // missing ones itself -- the bits their owner publishes -- then the batch is
                    // read again.
                    const int nq = nw / 2;
                    for (int q0 = wu * kWave; q0 < nq; q0 += kThreads) {
                        const int q = q0 + lane, i = 2 * q;
                        bool m = false;
                        if (q < nq && (i % 4 < 2 || (!kGreedy && rule != kRuleDeterministic && info[r0 + i / rw] != 0)))
                            m = static_cast<uint32_t>(load_word(src + i) >> 32) != tag ||
                                static_cast<uint32_t>(load_word(src + i + 1) >> 32) != tag;
                        for (uint64_t mask = __ballot(m); mask; mask &= mask - 1) {
                            const int iw = 2 * (q0 + __builtin_ctzll(mask));
                            const int row = r0 + iw / rw, c = (iw % rw) / 4, side = (iw % 4) / 2;
                            const int lo = c * kItem;
                            uint32_t w0, w1;
                            uint4 unused[kWaveLoads];
                            item_stats<T, kGreedy, kVecOK, true>((side ? draft : target) + (seq + row) * V, lo,
                                                                 min(V, lo + kItem), lane, k, unused, false, w0, w1);
                            if (lane == 0) {
                                put_word(src + iw, w0, tag);
                                put_word(src + iw + 1, w1, tag);
                            }
                        }
                    }
                    __threadfence();       // (this workgroup's stores have reached the device cache)
                    __syncthreads();
                    if (t == 0) {
                        s_late = 0;
                        __hip_atomic_fetch_add(ctl + 1, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    __syncthreads();
                    r0 -= rb;
                    continue;
                }
                // wave-uniform loop over groups of rpw rows; lane group `sub` owns one row
                for (int k0 = w * rpw; k0 < nr; k0 += kWaves * rpw) {
                    const int rl = k0 + sub;
                    const bool ok = rl < nr;
                    const int v = r0 + rl;
                    const float* sv = seg + (ok ? rl : 0) * rw;
                    if (kGreedy) {
                        float bv = -INFINITY;
                        int bi = INT_MAX;
                        if (ok)
                            for (int c = cl; c < nchunk; c += g)
                                argmax_merge(bv, bi, sv[c * 4], __float_as_int(sv[c * 4 + 1]));
                        for (int o = g >> 1; o > 0; o >>= 1) {
                            const float v2 = __shfl_xor(bv, o);
                            const int i2 = __shfl_xor(bi, o);
                            argmax_merge(bv, bi, v2, i2);
                        }
                        if (ok && cl == 0) info[v] = (bi >= 0 && bi < V) ? bi : 0;
                    } else {
                        const bool dr = ok && rule != kRuleDeterministic && info[v] != 0;
                        float mt = -INFINITY, md = -INFINITY;
                        if (ok)
                            for (int c = cl; c < nchunk; c += g) {
                                mt = fmaxf(mt, sv[c * 4]);
                                if (dr) md = fmaxf(md, sv[c * 4 + 2]);
                            }
                        for (int o = g >> 1; o > 0; o >>= 1) {
                            mt = fmaxf(mt, __shfl_xor(mt, o));
                            md = fmaxf(md, __shfl_xor(md, o));
                        }
                        double st = 0.0, sd = 0.0;
                        if (ok)
                            for (int c = cl; c < nchunk; c += g) {
                                const float x0 = sv[c * 4], x1 = sv[c * 4 + 1];
                                st += static_cast<double>(x1) * __builtin_amdgcn_exp2f(x0 - mt);
                                if (dr) {
                                    const float y0 = sv[c * 4 + 2], y1 = sv[c * 4 + 3];
                                    sd += static_cast<double>(y1) * __builtin_amdgcn_exp2f(y0 - md);
                                }
                            }
                        for (int o = g >> 1; o > 0; o >>= 1) {
                            st += __shfl_xor(st, o);
                            sd += __shfl_xor(sd, o);
                        }
                        if (ok && cl == 0) {
                            Mt[v] = mt; St[v] = st;
                            Md[v] = md; Sd[v] = sd;
                        }
                    }
                }
                __syncthreads();
            }
        }

        // -- E. per node: p, q of its token under its parent's rows, the ratio, its two uniforms
        asm volatile("" : "+v"(gzt), "+v"(gzd));
        for (int v = t; v < n1; v += kThreads) {
            float pv_ = NAN, qv_ = NAN;
            if (!kGreedy) {
                if (v > 0) {
                    const int pa = par[v];
                    const float zt = (v == t) ? widen<T>(gzt) : Elem<T>::load(target + (seq + SPECV_CHK(pa, n1, kSiteAcceptGatherRow)) * V,
                                                                                  SPECV_CHK(tok[v], V, kSiteAcceptGatherToken));
                    const double lp = static_cast<double>(zt) * k - Mt[pa];     // (log2 units)
                    const double pd = exp2(lp) / St[pa];
                    pv_ = static_cast<float>(pd);
                    if (rule == kRuleDeterministic) {
                        // a point-mass proposal: the ratio is p(x) itself (over the unrejected mass)
                        pq[v] = pd;
                        qx[v] = 1.f;
                    } else {
                        const float zd = (v == t) ? widen<T>(gzd) : Elem<T>::load(draft + (seq + SPECV_CHK(pa, n1, kSiteAcceptGatherRow)) * V,
                                                                                     SPECV_CHK(tok[v], V, kSiteAcceptGatherToken));
                        const double lq = static_cast<double>(zd) * k - Md[pa];
                        const double qd = exp2(lq) / Sd[pa];
                        pq[v] = exp2(lp - lq) * (Sd[pa] / St[pa]);
                        qx[v] = static_cast<float>(qd);
                        qv_ = static_cast<float>(qd);
                    }
                }
            }
            if (rank == 0) {
                if (p_tok) p_tok[seq + v] = pv_;
                if (q_tok) q_tok[seq + v] = qv_;
            }
        }
        __syncthreads();

        // -- F. the walk (wave 0; identical in every workgroup of the team); residual-mass passes
        //       are split over the team
        uint4 rt[kPassBatch], rd[kPassBatch];
        int npass = 0;
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
                            if (lane == 0) path[SPECV_CHK(n, n1, kSiteAcceptPath)] = c;
                            ++n;
                            v = c;
                            continue;
                        }
                        if (nxt < 0) { cmd = 1; break; }
                        const int c = nxt;
                        nxt = nsib[c];
                        // a repeated token: skipped when siblings are distinct draws (its test
                        // cannot pass and, without replacement or as a fixed candidate, changes
                        // nothing); an independent draw is tested like any other
                        if (dup[c] && rule != kRuleIid) continue;
                        // deterministic siblings: cs holds the rejected candidates' p mass and
                        // the target is p without them, renormalised
                        const double ratio = (rule == kRuleDeterministic)
                                                 ? (cs < 1.0 ? pq[c] / (1.0 - cs) : pq[c])
                                                 : fmax(0.0, pq[c] - cs) * Q / R;
                        if (uacc[c] < ratio) {
                            if (lane == 0) path[SPECV_CHK(n, n1, kSiteAcceptPath)] = c;
                            ++n;
                            v = c;
                            cs = 0.0; R = 1.0; Q = 1.0;
                            nxt = fch[v] < n1 ? fch[v] : -1;
                            continue;
                        }
                        if (rule == kRuleDeterministic) {
                            cs += pq[c];
                            continue;       // no residual pass: the draw excludes the rejected tokens
                        }
                        const double cn = cs + R / Q;
                        if (rule == kRuleWithoutReplacement) Q -= static_cast<double>(qx[c]);
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
                            s_qs = (cs > 0.0 && rule != kRuleDeterministic) ? static_cast<float>(cs / Sd[v]) : 0.f;
                            // deterministic siblings: the draw excludes every child's token (all
                            // were rejected, or repeat a rejected one); the list reuses ilist
                            int ne = 0;
                            if (rule == kRuleDeterministic)
                                for (int c = fch[v] < n1 ? fch[v] : -1; c >= 0; c = nsib[c]) ilist[ne++] = tok[c];
                            s_nexcl = ne;
                        }
                    }
                }
                __syncthreads();
                if (s_cmd != 0) break;
                const int64_t rr = (seq + SPECV_CHK(s_row, n1, kSiteAcceptEnd)) * V;
                const int row = s_row;
                const float ps = s_ps, qs = s_qs;
                const double mine = range_pass<T, kVecOK>(target + rr, draft + rr, V, my_t0, my_t1, Mt[row], Md[row],
                                                          k, ps, qs, ilist, 0, nullptr, red, rt, rd);
                double Rn = mine;
                if (P > 1) {
                    uint64_t* slots = pw + static_cast<int64_t>(SPECV_CHK(npass, n1 + 1, kSiteAcceptPass)) * P * 2;
                    // teammates whose share did not come in time: computed here
                    for (uint64_t miss = exchange_post(slots, P, rank, mine, tag, wait_ticks, s_vals, &s_mask); miss;
                         miss &= miss - 1) {
                        const int r = __builtin_ctzll(miss);
                        const int a0 = min(ntile, r * tpb), a1 = min(ntile, a0 + tpb);
                        exchange_fill(slots, r,
                                      range_pass_lean<T, kVecOK>(target + rr, draft + rr, V, a0, a1, Mt[row], Md[row], k,
                                                                 ps, qs, ilist, 0, red),
                                      tag, s_vals, ctl + 2);
                    }
                    double before_unused;
                    exchange_sum(s_vals, P, rank, before_unused, Rn);
                }
                ++npass;
                __syncthreads();
                if (t == 0) s_R = Rn;
                __syncthreads();
            }
        }

        // -- G. outputs of the walk (rank 0 of the team)
        const int cmd = s_cmd, e = s_row, na = s_n;
        if (rank == 0) {
            for (int i = t; i < n1; i += kThreads) {
                out_nodes[seq + i] = (i < na) ? path[i] : -1;
                if (i < na) out_tokens[seq + i] = tok[path[i]];
                else if (i > na) out_tokens[seq + i] = -1;
            }
            if (t == 0) accept_len[b] = na;
        }
        if (cmd == 2) {
            if (rank == 0 && t == 0) out_tokens[seq + SPECV_CHK(na, n1, kSiteAcceptOut)] = info[e];
            __syncthreads();
            continue;
        }

        // -- H. the draw at node e: w(x) = (p(x) - c q(x))+, smallest x whose CDF exceeds u * W
        const int64_t rr = (seq + SPECV_CHK(e, n1, kSiteAcceptEnd)) * V;
        const float mt = Mt[e], ps = s_ps, qs = s_qs;
        const float md = (qs != 0.f) ? Md[e] : 0.f;
        const int nexcl = s_nexcl;
        const double mine = range_pass<T, kVecOK>(target + rr, draft + rr, V, my_t0, my_t1, mt, md, k, ps, qs,
                                                  ilist, nexcl, seg, red, rt, rd);
        double before = 0.0, W = mine;
        if (P > 1) {
            uint64_t* slots = pw + static_cast<int64_t>(SPECV_CHK(npass, n1 + 1, kSiteAcceptPass)) * P * 2;
            for (uint64_t miss = exchange_post(slots, P, rank, mine, tag, wait_ticks, s_vals, &s_mask); miss;
                 miss &= miss - 1) {
                const int r = __builtin_ctzll(miss);
                const int a0 = min(ntile, r * tpb), a1 = min(ntile, a0 + tpb);
                exchange_fill(slots, r,
                              range_pass_lean<T, kVecOK>(target + rr, draft + rr, V, a0, a1, mt, md, k, ps, qs, ilist,
                                                         nexcl, red),
                              tag, s_vals, ctl + 2);
            }
            exchange_sum(s_vals, P, rank, before, W);
        }
        const double thr = ures[e] * W;
        // the owner: the first rank whose running sum passes thr (or, if rounding left thr at or
        // above the total, the last rank with mass); every workgroup finds the same one
        int owner = -1;
        if (W > 0.0) {
            if (P > 1) {
                double acc = 0.0;
                int lastpos = -1;
                for (int r = 0; r < P; ++r) {
                    if (s_vals[r] > 0.0) lastpos = r;
                    if (owner < 0 && acc + s_vals[r] > thr) owner = r;
                    acc += s_vals[r];
                }
                if (owner < 0) owner = lastpos;
            } else {
                owner = 0;
            }
        }
        if (owner == rank) {
            const int nseg = (my_t1 - my_t0) * kWaves;
            if (w == 0) {
                int sel = -1;
                double base = 0.0;
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
                const uint64_t hit = __ballot(s1 > s0 && before + incl > thr);
                int L;
                bool crossing;
                if (hit) {
                    L = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                    crossing = true;
                } else {
                    const uint64_t nz = __ballot(gs > 0.0);
                    L = nz ? 63 - __clzll(static_cast<long long>(nz)) : -1;
                    crossing = false;
                }
                if (L >= 0 && lane == L) {
                    double acc = before + incl - gs;
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
                if (lane == 0) {
                    s_sel = sel;
                    s_base = base;
                    s_found = -1;
                }
            }
            __syncthreads();
            const int sel = s_sel;
            if (sel >= 0 && w == sel % kWaves) {
                const int tl = sel / kWaves;                 // tile within this workgroup's range
                const int base = (my_t0 + tl) * kTile + (w * kWave + lane) * kVec;
                float zt[kVec], zd[kVec], wt[kVec];
#pragma unroll
                for (int i = 0; i < kVec; ++i) { zt[i] = -INFINITY; zd[i] = -INFINITY; }
                if (kVecOK && my_t1 - my_t0 <= kPassBatch) {
                    uint4 a = rt[0], c = rd[0];
#pragma unroll
                    for (int j = 1; j < kPassBatch; ++j)
                        if (j == tl) { a = rt[j]; c = rd[j]; }
                    if (base < V) {
                        cvt_vec<T>(a, zt);
                        if (qs != 0.f) cvt_vec<T>(c, zd);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < kVec; ++i)
                        if (base + i < V) {
                            zt[i] = Elem<T>::load(target + rr, base + i);
                            if (qs != 0.f) zd[i] = Elem<T>::load(draft + rr, base + i);
                        }
                }
                const uint32_t xm = excluded_in(ilist, nexcl, base);
                float ls = 0.f;
#pragma unroll
                for (int i = 0; i < kVec; ++i) {
                    wt[i] = ((xm >> i) & 1u) ? 0.f : draw_weight(zt[i], zd[i], mt, md, k, ps, qs);
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
            if (t == 0) out_tokens[seq + SPECV_CHK(na, n1, kSiteAcceptOut)] = (s_found >= 0 && s_found < V) ? s_found : 0;
        } else if (owner < 0 && rank == 0) {
            // no residual mass at all (a zero-probability event in exact arithmetic): the token with
            // the largest p(x) - c q(x), lowest index on ties
            float bv = -INFINITY;
            int bi = INT_MAX;
            for (int x = t; x < V; x += kThreads) {
                const float zt = Elem<T>::load(target + rr, x);
                const float zd = (qs != 0.f) ? Elem<T>::load(draft + rr, x) : -INFINITY;
                const float d = __builtin_amdgcn_exp2f(__builtin_fmaf(zt, k, -mt)) * ps -
                                __builtin_amdgcn_exp2f(__builtin_fmaf(zd, k, -md)) * qs;
                argmax_merge(bv, bi, d, x);
            }
            wave_argmax(bv, bi);
            if (lane == 0) { pv[w] = bv; pi[w] = bi; }
            __syncthreads();
            if (t == 0) {
                for (int i = 1; i < kWaves; ++i) argmax_merge(pv[0], pi[0], pv[i], pi[i]);
                out_tokens[seq + SPECV_CHK(na, n1, kSiteAcceptOut)] = (pi[0] >= 0 && pi[0] < V) ? pi[0] : 0;
            }
        }
        __syncthreads();
    }
    if (blockIdx.x == 0) {      // (every workgroup reaches A of its first sequence: these waits end)
        for (int i = t; i < static_cast<int>(gridDim.x); i += kThreads)
            while (__hip_atomic_load(seen + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag)
                __builtin_amdgcn_s_sleep(1);
        __syncthreads();
        if (t == 0) __hip_atomic_store(ctl, static_cast<uint64_t>(tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------------- host side


int team_size(int B) {
    const int cus = device_cu_count();
    return std::max(1, std::min(2, std::min(kMaxTeam, cus / std::max(B, 1))));
}

template <typename T>
int chunks_of(int V) { return (V + item_elems<T>() - 1) / item_elems<T>(); }

// How long a workgroup waits for a teammate's values before computing them itself: 100 us, or
// SPECV_ACCEPT_WAIT_US (microseconds; 0 makes every wait that is not already over compute the
// values here, which the tests use to run that path).
uint64_t wait_ticks() {
    const char* e = std::getenv("SPECV_ACCEPT_WAIT_US");
    long us = 100;
    if (e && *e) {
        char* end = nullptr;
        const long v = std::strtol(e, &end, 10);
        if (end && *end == '\0' && v >= 0 && v <= 10000000) us = v;
    }
    return static_cast<uint64_t>(us) * 100u;      // the wall clock runs at 100 MHz
}

// Whether phase 1 runs as a launch of its own before the team kernel: SPECV_ACCEPT_SPLIT = 0
// (never) or 1 (always); by default when the team kernel would deal at least kSplitItems items
// to each of its workgroups.  There the static deal's uneven finish costs more than the second
// launch (many sequences per team, or long rows over small teams); with a few items per
// workgroup the statistics hide under the team kernel's own start-up and the second launch is
// pure latency.
constexpr int64_t kSplitItems = 64;
bool split_stats(int64_t items, int grid) {
    const char* e = std::getenv("SPECV_ACCEPT_SPLIT");
    if (e && e[0] == '0' && e[1] == '\0') return false;
    if (e && e[0] == '1' && e[1] == '\0') return true;
    return items >= kSplitItems * grid;
}

template <typename T, bool kGreedy, bool kVecOK>
hipError_t launch_kernel(const AcceptArgs& a, hipStream_t stream) {
    int nchunk = chunks_of<T>(a.V);
    int P = team_size(a.B);
    const AcceptLayout lay(a.B, a.n1, nchunk, P);
    char* ws = static_cast<char*>(a.workspace);
    uint64_t* ctl = reinterpret_cast<uint64_t*>(ws + lay.ctl);
    uint32_t* seen = reinterpret_cast<uint32_t*>(ws + lay.seen);
    uint64_t* statw = reinterpret_cast<uint64_t*>(ws + lay.stat);
    uint64_t* partw = reinterpret_cast<uint64_t*>(ws + lay.part);
    const void* fn = reinterpret_cast<const void*>(&accept_kernel<T, kGreedy, kVecOK>);
    static std::atomic<int> occupancy[64];
    const int per_cu = cached_per_device(occupancy, [fn](int) {
        int nb = 0;
        return (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, 0) == hipSuccess && nb > 0) ? nb : 1;
    });
    const int capacity = per_cu * device_cu_count();
    const int nteams = std::max(1, std::min(a.B, capacity / P));
    const int grid = nteams * P;

    const T* target = static_cast<const T*>(a.target);
    const T* draft = static_cast<const T*>(a.draft);
    int B = a.B, n1 = a.n1, V = a.V;
    double invT = kGreedy ? 0.0 : 1.0 / static_cast<double>(a.temperature);
    float k = kGreedy ? 0.f : static_cast<float>(1.4426950408889634 * invT);   // log2(e) / T
    uint64_t seed = a.seed, offset = a.offset;
    uint64_t wt = wait_ticks();
    const int32_t* tokens = a.tokens;
    const int32_t* parent = a.parent;
    int32_t* accept_len = a.accept_len;
    int32_t* out_tokens = a.out_tokens;
    int32_t* out_nodes = a.out_nodes;
    float* p_tok = a.p_tok;
    float* q_tok = a.q_tok;
    int rule = a.rule;
    const int with_draft = (!kGreedy && rule != kRuleDeterministic) ? 1 : 0;
    const int64_t items = static_cast<int64_t>(B) * n1 * nchunk * (1 + with_draft);
    int stats_ready = 0;
    if (split_stats(items, grid)) {
        const int64_t wgs = std::min<int64_t>((items + kStatWaves - 1) / kStatWaves, int64_t{1} << 22);
        hipLaunchKernelGGL((accept_stats_kernel<T, kGreedy, kVecOK>), dim3(static_cast<unsigned>(wgs)),
                           dim3(kStatThreads), 0, stream, target, draft, parent, B, n1, V, nchunk, with_draft, k,
                           ctl, statw);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        stats_ready = 1;
    }
    hipLaunchKernelGGL((accept_kernel<T, kGreedy, kVecOK>), dim3(grid), dim3(kThreads), 0, stream, target, draft,
                       tokens, parent, B, n1, V, nchunk, P, rule, k, seed, offset, stats_ready, ctl, seen, wt,
                       statw, partw, accept_len, out_tokens, out_nodes, p_tok, q_tok);
    return hipGetLastError();
}

template <typename T, bool kVecOK>
hipError_t launch_typed(const AcceptArgs& a, hipStream_t stream) {
    if (a.temperature == 0.f) return launch_kernel<T, true, kVecOK>(a, stream);
    return launch_kernel<T, false, kVecOK>(a, stream);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

size_t accept_workspace_bytes(int B, int n1, int V, bool bf16) {
    const int nchunk = bf16 ? chunks_of<uint16_t>(V) : chunks_of<float>(V);
    return AcceptLayout(B, n1, nchunk, team_size(B)).total;
}

// The built-in workspace of the allocation-free entry point: zero when the library is loaded (the
// epoch words then hold 0), kept valid by the calls that use it.  One copy per device, held until
// the process ends; calls that overlap on one device race on it.
namespace {
static __device__ __align__(256) unsigned char scratch[kAcceptScratchBytes];
}  // namespace

hipError_t accept_scratch(void** ptr) {
    // the array's device address on the current device (the host-side name of the array is not
    // a device address), looked up once per device
    static std::atomic<void*> addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
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
