// spec_verify.hip -- HIP kernels for CDNA4 (gfx950) and the C ABI of the speculative
// decoding verify library (include/spec_verify.h).
//
// The verify calls walk each request (position by position, or node by node in a tree)
// and stop where the method stops, so they read only the rows it consults:
//   k_greedy_walk   greedy chain verify: a cluster of workgroups per request, each owning
//                   whole fine chunks of every row; per position the slices' argmax
//                   travels between the cluster's workgroups as tagged 64-bit atomic
//                   words (no fence), and every member takes the same decision.
//   k_chain_walk    chain rejection sampling, the same way with (max, exp-sum) per slice;
//                   after the stop each member weighs its slice of the row the last token
//                   is drawn from, and the cluster draws it (k_draw does when a slice
//                   spans more than 64 fine chunks).
//   k_tree_walk     the target-only tree walk (greedy or sampling), node by node.
//   k_mss_walk      the tree walk by multi-step speculative sampling with draft rows;
//                   a residual pass and a hand-off per rejected child.
//   k_draw          one wave per request: locates the chunk, then the segment, then the
//                   token holding u * total (inverse CDF in ascending token id).
// The eager passes read every row and hand over at kernel boundaries; they are selected
// with spec_options.path = SPEC_PATH_EAGER (the filtered chain always reads every row):
//   k_rows          streams every target-logit row once from HBM (16-byte non-temporal
//                   buffer loads, two batches of kUnroll per lane in flight), split over `S`
//                   workgroups per row.  Each workgroup reduces its chunk to one 16-byte
//                   record: the chunk max, the lowest index attaining it (greedy) and
//                   sum exp((l - m)/T) relative to the chunk max (sampling).
//   k_greedy_merge  one workgroup per request: row argmax from the records, first
//                   mismatch with the drafts, emitted tokens.
//   k_tree          one workgroup per request: validates the parent array (pointer
//                   jumping for depths), row statistics of every node and the target
//                   probability of every node's token, then the level-by-level walk; it
//                   hands the row and the excluded tokens of the last draw to k_mass.
//   k_chain_accept  one workgroup per chain request: row max and normaliser from the
//                   records, p(x_i) / q(x_i) tests in fp64, the accepted prefix, and the
//                   state of the last draw (correction from row k, or bonus from row G).
//   k_mass          one workgroup per (request, fine chunk of 4096 elements): weight of
//                   the chunk and of each of its 64 segments of 64 elements in the row the
//                   last token is drawn from.
// An agent-scope fence inside a kernel writes back and invalidates the whole L2 of an
// XCD, so no kernel uses one.
//
// Sources: llm-infra-atlas "Speculative Decoding" section 0 and section 2; ricardokevins
// "Speculative Decoding", correction sampling, Eq. a(x) and Eq. r(x); zdszero
// "spec_origins": Blockwise Parallel Decoding (verify), Speculative Decoding (acceptance
// rule items 1-3), SpecInfer, and "in SGLang" (target-only tree walk).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "spec_verify.h"

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kUnroll = 4;
constexpr int kWalkUnroll = 4;  // loads per lane and batch in the walks' row passes
constexpr int kMaxSplits = 64;
constexpr long kChunkBytes = 64 * 1024;  // target logit bytes per row-pass workgroup
constexpr int kFine = 4 * 4 * kBlock;  // elements per fine chunk of the final draw (4096)
constexpr int kSeg = 64;               // elements per segment: one per lane of a wave
constexpr int kSegs = kFine / kSeg;    // segments per fine chunk (64)
constexpr int kMaxRows = SPEC_MAX_G + 1;
constexpr float kLog2e = 1.44269504088896340736f;


// One record per (row, split): chunk max, lowest index attaining it, and the chunk's
// sum of exp2((l - m) * log2(e) / T) relative to that max (sampling only).
struct alignas(16) Part {
    float m;
    int idx;
    double z;
};

// What the last token of a request is drawn from, handed from the acceptance scan (chain)
// or the walk (tree) to k_mass and k_draw.  Every call writes it for every request.
enum DrawKind { kDrawNone = -1, kDrawResidual = 0, kDrawTarget = 1 };
struct alignas(16) DrawState {
    int kind;    // kDrawNone: nothing to draw (invalid request, greedy tree)
    int row;     // logit row b * R + k (chain) or b * N + cur (tree)
    int qrow;    // kDrawResidual: q row b * G + k (chain), b * N + cur (tree with q)
    int out;     // index of the drawn token in out_tokens / probs_out
    int coin;    // index of its coin in coins
    int nexcl;   // tree: distinct tokens of the children tried last, in excl[b][...]
    float M;     // row max
    float invZ;  // 1 / Z rounded to fp32 (weights)
    double Z;    // sum exp((l - M) / T) over the (kept part of the) row
    double T;    // temperature
    uint32_t thp;  // filtered calls: target tokens whose order key is below thp weigh 0
    uint32_t thq;  // filtered residual: the same for the draft row qrow of draft_logits
    float Mq;      // filtered residual: draft row max
    float invZq;   // filtered residual: 1 / kept draft mass
    float cq;      // kDrawResidual: weights max(0, p - cq * q) (1 for the chain)
};

// Field-wise store of a draw state (to global memory or LDS).  A whole-struct copy of a state that
// the kernel also passes by reference becomes a private array of its zero fields, which the
// compiler may move into LDS (3 KiB per workgroup); in the tree walk that array cost tree
// sampling 10 us, with residency unchanged.
__device__ inline void store_state(DrawState* p, const DrawState& st) {
    p->kind = st.kind;
    p->row = st.row;
    p->qrow = st.qrow;
    p->out = st.out;
    p->coin = st.coin;
    p->nexcl = st.nexcl;
    p->M = st.M;
    p->invZ = st.invZ;
    p->Z = st.Z;
    p->T = st.T;
    p->thp = st.thp;
    p->thq = st.thq;
    p->Mq = st.Mq;
    p->invZq = st.invZq;
    p->cq = st.cq;
}

// Field-wise copy of a draw state (from global memory or LDS; keeps it in registers).
__device__ inline DrawState load_state(const DrawState* p) {
    DrawState st;
    st.kind = p->kind;
    st.row = p->row;
    st.qrow = p->qrow;
    st.out = p->out;
    st.coin = p->coin;
    st.nexcl = p->nexcl;
    st.M = p->M;
    st.invZ = p->invZ;
    st.Z = p->Z;
    st.T = p->T;
    st.thp = p->thp;
    st.thq = p->thq;
    st.Mq = p->Mq;
    st.invZq = p->invZq;
    st.cq = p->cq;
    return st;
}

// Top-k / top-p result of one logit row (filtered calls).
struct alignas(16) FiltRow {
    float M;       // row max (-inf: the row has no finite logit)
    uint32_t th;   // tokens whose order key is below th are removed (0: none)
    double Z;      // kept mass: sum of exp((l - M) / T) over the kept tokens
};

struct KArgs {
    const void* logits;
    const float* q;
    const int32_t* tokens;  // chain: draft tokens [B][G]; tree: node tokens [B][N]
    const int32_t* parents;
    const float* coins;
    const float* temperature;
    int B, R, V, S, chunk, D;
    int S2;              // fine chunks of kFine elements per row (final draw)
    float th_single, th_acc;
    int32_t* accept_len;
    int32_t* out_tokens;
    int32_t* accepted_nodes;
    float* probs;
    Part* parts;         // [rows][S] records of the row pass
    DrawState* dstate;   // [B]
    double* mass;        // [B][S2] draw weight of each fine chunk
    double* massfb;      // [B][S2] fallback weight (the plain target row)
    double* seg;         // [B][S2][kSegs] draw weight of each segment
    int32_t* excl;       // [B][SPEC_MAX_N] tree: excluded tokens of the final draw
    const void* dlogits; // filtered calls: draft logits [B][G][V]
    const int32_t* top_k;
    const float* top_p;
    FiltRow* frows;      // filtered calls: [B*R] target rows, then [B*G] draft rows
    int32_t* kept;       // filtered calls: per target row, [kBlock + 1] words: the count of
                         // tokens the filter keeps (-1: not listed), then their ids
    int fixbits;         // fixed-point fraction bits of the filter's mass histograms
    int walk_temporal;   // chain walk: row passes with cache-allocating loads (sweeps: 0)
    int coin_stride;     // coins per request in `coins`; the final draw's coin is the last
    int walk_draw;       // chain walk: the final draw happens in the walk (no k_draw)
    int spin;            // walks: polls before a hand-off wait gives up
    unsigned* hdr;       // workspace header: the walks' call counter and finished count
};

// ---------------------------------------------------------------------------------------
// element access

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load that does not displace reusable lines from the caches.
__device__ inline u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
// Buffer loads: the fourth word of a raw buffer resource (32-bit data format, no stride
// swizzle), and the cache-policy bit of a non-temporal load.
constexpr int kBufWord3 = 0x00020000;
constexpr int kCacheNT = 2;
// s_waitcnt immediate of vmcnt(n) alone, n < 64 (expcnt and lgkmcnt at their maxima; vmcnt's
// low four bits at 3:0, its high two at 15:14)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <typename T>
struct Ld;

template <>
struct Ld<float> {
    static constexpr int kVec = 4;
    __device__ static float one(const float* p) { return *p; }
    __device__ static void unpack(const u32x4& v, float* f) {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
};

template <>
struct Ld<uint16_t> {  // bf16 bit patterns: the value is the high half of an fp32
    static constexpr int kVec = 8;
    __device__ static float one(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
    __device__ static void unpack(const u32x4& v, float* f) {
        f[0] = __uint_as_float(v.x << 16);
        f[1] = __uint_as_float(v.x & 0xffff0000u);
        f[2] = __uint_as_float(v.y << 16);
        f[3] = __uint_as_float(v.y & 0xffff0000u);
        f[4] = __uint_as_float(v.z << 16);
        f[5] = __uint_as_float(v.z & 0xffff0000u);
        f[6] = __uint_as_float(v.w << 16);
        f[7] = __uint_as_float(v.w & 0xffff0000u);
    }
};

// ---------------------------------------------------------------------------------------
// wave64 / block reductions (butterfly: every lane ends with the same bits)

__device__ inline float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ inline double wave_sum(double v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ inline void arg_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

__device__ inline void wave_argmax(float& v, int& i) {
    for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(v, o);
        int i2 = __shfl_xor(i, o);
        arg_merge(v, i, v2, i2);
    }
}

// The split records of one request, staged in LDS by the per-request merges.
struct RecSmem {
    float m[kMaxRows * kMaxSplits];
    union {
        double z[kMaxRows * kMaxSplits];  // sampling: exp-sums
        int i[kMaxRows * kMaxSplits];     // greedy: argmax indices
    };
};

struct Smem {  // per-request merges: row statistics, drafts, coins, decisions
    float M[kMaxRows];
    double Z[kMaxRows];
    double p[kMaxRows];
    int arg[kMaxRows];
    int x[kMaxRows];
    float l[kMaxRows];
    float qx[kMaxRows];
    float u[kMaxRows];
    DrawState st;
    int k;
};

// ---------------------------------------------------------------------------------------
// the row pass of one chunk: per-thread streaming state, then a block reduction
//
// Each lane takes kU 16-byte vectors per batch, strided by the block so that every
// load instruction of the wave is one contiguous 1 KB segment.  Within a lane, batches
// arrive in ascending index order, and so do the vectors within a batch.
//   sampling: online (m, z): per batch the batch max, one rescale of z if it grew, then
//             sum exp2((l - m) * log2(e) / T) in fp32 over the batch, added to z in fp64.
//   greedy:   the running max and, when a batch raises it, the first element of that
//             batch equal to it (from the registers already loaded): the lane's lowest
//             index of its max, since a lane's elements arrive in index order.

struct RowSmem {
    float rm[kWaves];
    double rz[kWaves];
    int ri[kWaves];
};

// Block-wide max of v (every thread gets it).
__device__ inline float block_max(float v, RowSmem& sm) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max(v);
    if (lane == 0) sm.rm[wave] = v;
    __syncthreads();
    float r = sm.rm[0];
    for (int w = 1; w < kWaves; ++w) r = fmaxf(r, sm.rm[w]);
    return r;
}

// Block-wide min of v (every thread gets it).
__device__ inline int block_min(int v, RowSmem& sm) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    if (lane == 0) sm.ri[wave] = v;
    __syncthreads();
    int r = sm.ri[0];
    for (int w = 1; w < kWaves; ++w) r = min(r, sm.ri[w]);
    return r;
}

// Reduces chunk [c0, c1) of a row into one record (valid in every thread).  The loads of
// batch j + 1 (kU 16-byte vectors per lane) are issued before batch j is reduced, so the
// reduction's arithmetic overlaps the memory latency; that matters most when a workgroup
// has its SIMDs to itself, as in the walks' later positions.
//
// bkey (optional): batch j of this lane (its vectors v = tid +
// kBlock * (kU * j + u)) leaves the top 16 bits of its maximum's order key in
// bkey[j * kBlock + tid], for the first kMaxBatchRec batches.
constexpr int kMaxBatchRec = 24;
template <typename T, bool kSampling, bool kNT = true, int kU = kUnroll>
__device__ __attribute__((always_inline)) Part chunk_record(const T* rowp, int c0, int c1,
                                                            float s2, RowSmem& sm,
                                                            float* lane_max = nullptr,
                                                            uint16_t* bkey = nullptr) {
    constexpr int kVec = Ld<T>::kVec;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = c1 > c0 ? c1 - c0 : 0;
    const T* p = rowp + c0;
    int head = (int)(((16u - ((uint32_t)(uintptr_t)p & 15u)) & 15u) / sizeof(T));
    if (head > n) head = n;
    const int nv = (n - head) / kVec;
    const int tail0 = head + nv * kVec;
    const u32x4* vp = reinterpret_cast<const u32x4*>(p + head);
    const int ebase = c0 + head;  // row index of the first vector element

    float m = -INFINITY;   // running max (sampling: reference of z)
    double z = 0.0;        // sampling: sum exp2((l - m) * s2)
    int im = INT_MAX;      // greedy: lowest index attaining m among this lane's vectors
    float ms = -INFINITY;  // greedy: max over this lane's scalar head / tail elements
    int is = INT_MAX;      //         lowest index attaining ms

    auto scalar = [&](int e) {  // one element at chunk offset e (head or tail)
        const float x = Ld<T>::one(p + e);
        if (kSampling) {
            if (x > m) {
                z *= (double)ex2((m - x) * s2);
                m = x;
            }
            if (m != -INFINITY) z += (double)ex2((x - m) * s2);
        } else if (x > ms) {
            ms = x;
            is = c0 + e;
        }
    };
    // One batch of nvec 16-byte vectors, unpacked on the fly (once for the batch max, once
    // for the exp-sum) so that only the raw vectors stay live while the loads are in flight.
    auto batch = [&](u32x4* raw, int nvec, int vfirst) -> float {
        float bm;
        {
            float f[kVec];
            Ld<T>::unpack(raw[0], f);
            bm = f[0];
#pragma unroll
            for (int e = 1; e < kVec; ++e) bm = fmaxf(bm, f[e]);
        }
#pragma unroll
        for (int u = 1; u < nvec; ++u) {
            float f[kVec];
            Ld<T>::unpack(raw[u], f);
#pragma unroll
            for (int e = 0; e < kVec; ++e) bm = fmaxf(bm, f[e]);
        }
        if (kSampling) {
            if (bm > m) {
                z *= (double)ex2((m - bm) * s2);
                m = bm;
            }
            if (m != -INFINITY) {
                float acc = 0.f;
#pragma unroll
                for (int u = 0; u < nvec; ++u) {
                    // deep batches: unpack again rather than keep the first unpacking
                    // live (emits no code)
                    if constexpr (kU > 4) asm volatile("" : "+v"(raw[u]));
                    float f[kVec], e8[kVec];
                    Ld<T>::unpack(raw[u], f);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) e8[e] = ex2((f[e] - m) * s2);
                    float t;
                    if (kVec == 8)
                        t = ((e8[0] + e8[1]) + (e8[2] + e8[3])) + ((e8[4] + e8[5]) + (e8[6] + e8[7]));
                    else
                        t = (e8[0] + e8[1]) + (e8[2] + e8[3]);
                    acc += t;
                }
                z += (double)acc;
            }
        } else if (bm > m) {  // a new maximum: its first element in this batch (index order)
            m = bm;
            int first = INT_MAX;
#pragma unroll
            for (int u = nvec - 1; u >= 0; --u) {
                float f[kVec];
                Ld<T>::unpack(raw[u], f);
#pragma unroll
                for (int e = kVec - 1; e >= 0; --e)
                    if (f[e] == bm) first = (vfirst + u * kBlock) * kVec + e;
            }
            im = ebase + first;
        }
        return bm;
    };

    auto record = [&](float bm, int v0) {
        if (bkey) {
            const int j = (v0 - tid) / (kU * kBlock);
            // +0.0f: a -0.0 maximum stands for +0.0 too (fmaxf may return either)
            const uint32_t u = __float_as_uint(bm + 0.0f);
            if (j < kMaxBatchRec)
                bkey[j * kBlock + tid] = (uint16_t)(((u & 0x80000000u) ? ~u : (u | 0x80000000u)) >> 16);
        }
    };
    if (tid < head) scalar(tid);
    int v = tid;
    {
        // Two named buffers take turns, so no register copy waits for a load.  The loads are
        // buffer loads over the slice's nv vectors (the base in scalar registers, one 32-bit
        // offset per lane): a load past the end reads zeros and is discarded, so every load is
        // issued unconditionally (under a branch the compiler could not tell which loads are
        // outstanding and would wait for all of them), and no 64-bit per-lane address is kept
        // whose registers a load in flight could overwrite (the compiler then waited for that
        // load before computing the next address, once every two batches).  A lane's last
        // batch may be partial; its loads are in flight during the batch before it like any
        // other, and its vectors are reduced one by one in index order.
        const int step = kU * kBlock;
        auto full = [&](int v0) { return v0 + (kU - 1) * kBlock < nv; };
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, nv * 16, kBufWord3);
        auto loadc = [&](u32x4* raw, int v0) {
            // the whole offset in the lane's operand: the range check covers it (the scalar
            // offset would be added after the check)
#pragma unroll
            for (int u = 0; u < kU; ++u)
                raw[u] = __builtin_amdgcn_raw_buffer_load_b128(
                    rsrc, (int)((uint32_t)(v0 + u * kBlock) * 16u), 0, kNT ? kCacheNT : 0);
        };
        auto reduce = [&](u32x4* raw, int v0) {
            if (full(v0)) {
                record(batch(raw, kU, v0), v0);
            } else {
#pragma unroll
                for (int u = 0; u < kU; ++u)
                    if (v0 + u * kBlock < nv) batch(&raw[u], 1, v0 + u * kBlock);
            }
        };
        // Every thread runs the same number of batches (those of thread 0, which has the
        // most), so the loop is uniform; a thread's batches past its end are empty.  Before
        // a batch is reduced exactly the next batch's kU loads are still in flight, which
        // the explicit wait states for the compiler: otherwise it merges the paths where a
        // wave reduced nothing and waits at the top of the loop for every load (the
        // pipeline drained once every two batches).
        // (A loop over pairs of batches with no exit in between: an exit after the first of
        // a pair left a path back to the top, never taken, on which the compiler also
        // waited for every load.)
        const int nb = (nv + step - 1) / step;  // the same in every thread
        if (nb > 0) {
            u32x4 ra[kU], rb[kU];
            loadc(ra, v);
            for (int j = 0; j + 1 < nb; j += 2) {
                loadc(rb, v + step);
                __builtin_amdgcn_sched_barrier(0);  // batch j + 1 in flight before batch j is reduced
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(kU));
                reduce(ra, v);
                v += step;
                loadc(ra, v + step);  // past the last batch: zeros, discarded
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(kU));
                reduce(rb, v);
                v += step;
            }
            if (nb & 1) {  // the last batch, loaded by the pair before it (or first)
                reduce(ra, v);
                v += step;
            }
        }
    }
    if (tail0 + tid < n) scalar(tail0 + tid);

    Part r;
    if (kSampling) {  // block max, then every lane rescales its sum to it once
        if (lane_max) *lane_max = m;
        const float M = block_max(m, sm);
        double zz = 0.0;
        if (m != -INFINITY) zz = m == M ? z : z * (double)ex2((m - M) * s2);
        zz = wave_sum(zz);
        if (lane == 0) sm.rz[wave] = zz;
        __syncthreads();
        double Z = sm.rz[0];
        for (int w = 1; w < kWaves; ++w) Z += sm.rz[w];
        r.m = M;
        r.z = Z;
        r.idx = INT_MAX;
        return r;
    }
    const float M = block_max(fmaxf(m, ms), sm);
    int idx = INT_MAX;
    if (M != -INFINITY) {
        if (ms == M) idx = is;
        if (m == M) idx = min(idx, im);
    }
    r.m = M;
    r.idx = block_min(idx, sm);
    r.z = 0.0;
    return r;
}

// ---------------------------------------------------------------------------------------
// k_rows: one workgroup per (row, split)

template <typename T, bool kSampling>
__global__ __launch_bounds__(kBlock) void k_rows(KArgs a) {
    __shared__ RowSmem sm;
    const int S = a.S;
    const int blk = blockIdx.x;
    const int row = blk / S;
    const int s = blk - row * S;
    const int b = row / a.R;
    const T* rowp = reinterpret_cast<const T*>(a.logits) + (size_t)row * a.V;
    const int c0 = s * a.chunk;
    const int c1 = min(a.V, c0 + a.chunk);
    float s2 = 0.f;
    if (kSampling) s2 = kLog2e / a.temperature[b];
    // the pipelined pass: 64.5 against 66.8 us for the eager greedy call on the large batch
    const Part r = chunk_record<T, kSampling, true, kUnroll>(rowp, c0, c1, s2, sm);
    if (threadIdx.x == 0) a.parts[(size_t)row * S + s] = r;
}

// ---------------------------------------------------------------------------------------
// k_greedy_merge: one workgroup per request

template <typename T>
__global__ __launch_bounds__(kBlock) void k_greedy_merge(KArgs a) {
    __shared__ Smem sm;
    __shared__ RecSmem rs;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = a.R, G = R - 1, S = a.S;
    const int b = blockIdx.x;
    const Part* pr = a.parts + (size_t)b * R * S;
    for (int r = tid; r < R * S; r += kBlock) {  // records and drafts, all loads at once
        const Part p = pr[r];
        rs.m[r] = p.m;
        rs.i[r] = p.idx;
    }
    if (tid < G) sm.x[tid] = a.tokens[(size_t)b * G + tid];
    __syncthreads();
    for (int i = wave; i < R; i += kWaves) {  // row argmax (lowest index), one wave per row
        float v = -INFINITY;
        int ix = INT_MAX;
        if (lane < S) {
            v = rs.m[i * S + lane];
            ix = rs.i[i * S + lane];
        }
        wave_argmax(v, ix);
        if (lane == 0) sm.arg[i] = v == -INFINITY ? -1 : ix;
    }
    __syncthreads();
    if (tid == 0) {
        const int* x = sm.x;
        bool valid = true;  // only what the positions up to the first mismatch consult
        int k = G;
        for (int i = 0; i <= G; ++i) {
            if (sm.arg[i] < 0) {
                valid = false;
                break;
            }
            if (i == G) break;
            if (x[i] < 0 || x[i] >= a.V) {
                valid = false;
                break;
            }
            if (x[i] != sm.arg[i]) {
                k = i;
                break;
            }
        }
        sm.k = valid ? k : -1;
        a.accept_len[b] = sm.k;
    }
    __syncthreads();
    const int k = sm.k;
    for (int i = tid; i < R; i += kBlock) {
        int t = -1;
        if (k >= 0) t = i < k ? sm.x[i] : (i == k ? sm.arg[k] : -1);
        a.out_tokens[(size_t)b * R + i] = t;
    }
}

// Four consecutive target logits as one load (8 bytes of bf16 or 16 bytes of fp32).
template <typename T>
struct Quad;
template <>
struct Quad<float> {
    typedef u32x4 Raw;
    Raw raw;
    __device__ static void unpack(const Raw& r, float* l) {
        l[0] = __uint_as_float(r.x);
        l[1] = __uint_as_float(r.y);
        l[2] = __uint_as_float(r.z);
        l[3] = __uint_as_float(r.w);
    }
};
template <>
struct Quad<uint16_t> {
    typedef unsigned int Raw __attribute__((ext_vector_type(2)));
    Raw raw;
    __device__ static void unpack(const Raw& r, float* l) {
        l[0] = __uint_as_float(r.x << 16);
        l[1] = __uint_as_float(r.x & 0xffff0000u);
        l[2] = __uint_as_float(r.y << 16);
        l[3] = __uint_as_float(r.y & 0xffff0000u);
    }
};

// ---------------------------------------------------------------------------------------
// the acceptance scan of a chain request (block-wide; identical bits in every caller)
//
// Row max and normaliser from the records, p(x_i) / q(x_i) tests in fp64 with the
// request's coins, and the state of the final draw (the correction from row k, or the
// bonus from row G).  With `emit`, the accepted prefix, accept_len and probs are written.

template <typename T>
__device__ DrawState chain_accept(const KArgs& a, int b, bool emit, Smem& sm, RecSmem& rs) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = a.R, G = R - 1, S = a.S, V = a.V;
    const T* logits = reinterpret_cast<const T*>(a.logits);
    // every load of the request at once: records, coins, drafts, and the two gathers
    const Part* pr = a.parts + (size_t)b * R * S;
    for (int r = tid; r < R * S; r += kBlock) {
        const Part p = pr[r];
        rs.m[r] = p.m;
        rs.z[r] = p.z;
    }
    if (tid < R) sm.u[tid] = a.coins[(size_t)b * R + tid];
    if (tid < G) {
        const int xi = a.tokens[(size_t)b * G + tid];
        sm.x[tid] = xi;
        if (xi >= 0 && xi < V) {
            sm.l[tid] = Ld<T>::one(logits + ((size_t)b * R + tid) * V + xi);
            sm.qx[tid] = a.q[((size_t)b * G + tid) * V + xi];
        }
    }
    const float Tf = a.temperature[b];
    const bool t_ok = isfinite(Tf) && Tf > 0.f;
    const double Td = (double)Tf;
    __syncthreads();
    for (int i = wave; i < R; i += kWaves) {  // row max and normaliser, one wave per row
        float m = -INFINITY;
        double z = 0.0;
        if (lane < S) {
            m = rs.m[i * S + lane];
            z = rs.z[i * S + lane];
        }
        const float M = wave_max(m);
        double term = 0.0;
        if (lane < S && m != -INFINITY) term = z * exp(((double)m - (double)M) / Td);
        const double Z = wave_sum(term);
        if (lane == 0) {
            sm.M[i] = M;
            sm.Z[i] = Z;
        }
    }
    __syncthreads();
    if (tid < R) {  // lane i: is everything position i consults usable, and is x_i kept?
        bool ok = sm.M[tid] != -INFINITY && sm.u[tid] > 0.f && sm.u[tid] <= 1.f;
        bool keep = false;
        if (tid < G) {
            const int xi = sm.x[tid];
            ok = ok && xi >= 0 && xi < V;
            if (ok) ok = sm.qx[tid] >= 0.f && isfinite(sm.qx[tid]);
            if (ok && t_ok) {
                const double p = exp(((double)sm.l[tid] - (double)sm.M[tid]) / Td) / sm.Z[tid];
                const double qx = (double)sm.qx[tid];
                keep = qx > 0.0 ? (p > 0.0 && (double)sm.u[tid] <= p / qx) : p > 0.0;
                sm.p[tid] = p;
            }
        }
        sm.arg[tid] = (ok ? 1 : 0) | (keep ? 2 : 0);
    }
    __syncthreads();
    if (tid == 0) {  // positions in order up to the first rejection; the final coin always
        bool valid = t_ok && sm.u[G] > 0.f && sm.u[G] <= 1.f;
        int k = G;
        for (int i = 0; i <= G && valid; ++i) {
            if (!(sm.arg[i] & 1)) {
                valid = false;
                break;
            }
            if (i < G && !(sm.arg[i] & 2)) {
                k = i;
                break;
            }
        }
        sm.k = valid ? k : -1;
        if (emit) a.accept_len[b] = sm.k;
        DrawState st = {};
        st.kind = kDrawNone;
        if (valid) {
            st.kind = k < G ? kDrawResidual : kDrawTarget;
            st.row = b * R + k;
            st.qrow = b * G + k;
            st.out = b * R + k;
            st.coin = b * R + G;
            st.nexcl = 0;
            st.cq = 1.f;
            st.M = sm.M[k];
            st.Z = sm.Z[k];
            st.invZ = (float)(1.0 / sm.Z[k]);
            st.T = Td;
        }
        store_state(&sm.st, st);
    }
    __syncthreads();
    const DrawState st = load_state(&sm.st);
    const int k = sm.k;
    for (int i = tid; i < R && emit; i += kBlock) {
        int t = -1;
        float pr2 = 0.f;
        if (k >= 0 && i < k) {
            t = sm.x[i];
            pr2 = (float)sm.p[i];
        }
        if (i != k) {  // slot k is written by the final draw
            a.out_tokens[(size_t)b * R + i] = t;
            if (a.probs) a.probs[(size_t)b * R + i] = pr2;
        }
    }
    __syncthreads();  // sm is reused by the caller
    return st;
}

// ---------------------------------------------------------------------------------------
// k_tree: one workgroup per request

struct TreeSmem {
    int par[SPEC_MAX_N];
    int tok[SPEC_MAX_N];
    union {
        struct {  // validation: pointer-jumping state
            int anc[SPEC_MAX_N];
            int dep[SPEC_MAX_N];
        };
        struct {  // the walk: children of the current node, tokens to exclude
            int kids[SPEC_MAX_N];
            int excl[SPEC_MAX_N];
        };
    };
    float M[SPEC_MAX_N];     // row max
    int arg[SPEC_MAX_N];     // greedy: row argmax (lowest id), -1 if no finite logit
    double Z[SPEC_MAX_N];    // sampling: sum exp((l - M) / T) over the row
    double pc[SPEC_MAX_N];   // sampling: p_parent(token of node c), by node id
    int wcnt[kWaves];
    int chosen;
};

// Statistics of all N rows of request b from their records, g = 2^ceil(log2 S) lanes per
// row, 64 / g rows per wave at a time.  The butterflies use only xor offsets below g, so
// the sums are the same bits as a full-wave butterfly with zero padding.
__device__ void tree_row_stats(const KArgs& a, int b, bool sampling, double Td, TreeSmem& ts) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int S = a.S, N = a.R;
    int g = 1;
    while (g < S) g <<= 1;
    const int per_wave = 64 / g;
    const int sub = lane / g, s = lane - sub * g;
    for (int j0 = wave * per_wave; j0 < N; j0 += kWaves * per_wave) {  // uniform per wave
        const int j = j0 + sub;
        const bool have = j < N && s < S;
        float m = -INFINITY;
        int ix = INT_MAX;
        double z = 0.0;
        if (have) {
            const Part pr = a.parts[((size_t)b * N + j) * S + s];
            m = pr.m;
            ix = pr.idx;
            z = pr.z;
        }
        if (sampling) {
            float M = m;
            for (int o = g >> 1; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
            double term = (have && m != -INFINITY) ? z * exp(((double)m - (double)M) / Td) : 0.0;
            for (int o = g >> 1; o > 0; o >>= 1) term += __shfl_xor(term, o);
            if (s == 0 && j < N) {
                ts.M[j] = M;
                ts.Z[j] = term;
            }
        } else {
            for (int o = g >> 1; o > 0; o >>= 1) {
                const float v2 = __shfl_xor(m, o);
                const int i2 = __shfl_xor(ix, o);
                arg_merge(m, ix, v2, i2);
            }
            if (s == 0 && j < N) {
                ts.M[j] = m;
                ts.arg[j] = m == -INFINITY ? -1 : ix;
            }
        }
    }
    __syncthreads();
}

// Depth of every node by pointer jumping (parents[i] < i, so every chain of parents ends
// at the root): ceil(log2 N) rounds.  par, anc and dep are LDS arrays of N entries; the
// parent array must already be validated.  Block-wide.
template <int kThreads = kBlock>
__device__ void tree_depths(const int* par, int N, int* anc, int* dep) {
    const int tid = threadIdx.x;
    for (int i = tid; i < N; i += kThreads) {
        anc[i] = i == 0 ? 0 : par[i];
        dep[i] = i == 0 ? 0 : 1;
    }
    for (int r = 1; r < N; r <<= 1) {
        __syncthreads();
        int nd[SPEC_MAX_N / kThreads], na[SPEC_MAX_N / kThreads];
        int c = 0;
        for (int i = tid; i < N; i += kThreads, ++c) {
            const int an = anc[i];
            nd[c] = dep[i] + (an == i ? 0 : dep[an]);
            na[c] = anc[an];
        }
        __syncthreads();
        c = 0;
        for (int i = tid; i < N; i += kThreads, ++c) {
            if (anc[i] != i) {
                dep[i] = nd[c];
                anc[i] = na[c];
            }
        }
    }
    __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_tree(KArgs a, int sampling) {
    __shared__ TreeSmem ts;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const int N = a.R, V = a.V, D = a.D;
    const int32_t* par_g = a.parents + (size_t)b * N;
    const int32_t* tok_g = a.tokens + (size_t)b * N;
    const T* logits = reinterpret_cast<const T*>(a.logits);
    bool bad = false;
    for (int i = tid; i < N; i += kBlock) {
        const int p = par_g[i];
        const int t = tok_g[i];
        ts.par[i] = p;
        ts.tok[i] = t;
        if (i == 0) {
            if (p != -1) bad = true;
        } else {
            if (p < 0 || p >= i) bad = true;
            if (t < 0 || t >= V) bad = true;
        }
    }
    float Tf = 1.f;
    if (sampling) {
        Tf = a.temperature[b];
        if (!(isfinite(Tf) && Tf > 0.f)) bad = true;
        for (int d = tid; d <= D; d += kBlock) {
            const float u = a.coins[(size_t)b * (D + 1) + d];
            if (!(u > 0.f && u <= 1.f)) bad = true;
        }
    }
    const double Td = (double)Tf;
    bad = __syncthreads_or(bad);
    if (!bad) {
        tree_depths(ts.par, N, ts.anc, ts.dep);
        for (int i = tid; i < N; i += kBlock)
            if (ts.dep[i] > D) bad = true;
        // every row's statistics (a row the walk reaches needs a finite logit)
        tree_row_stats(a, b, sampling != 0, Td, ts);
        bad = __syncthreads_or(bad);
    }
    int32_t* out = a.out_tokens + (size_t)b * (D + 1);
    int32_t* nodes = a.accepted_nodes + (size_t)b * D;
    float* probs = a.probs ? a.probs + (size_t)b * (D + 1) : nullptr;
    if (bad) {
        for (int d = tid; d <= D; d += kBlock) {
            out[d] = -1;
            if (d < D) nodes[d] = -1;
            if (probs) probs[d] = 0.f;
        }
        if (tid == 0) {
            a.accept_len[b] = -1;
            if (sampling) {
                DrawState st = {};
                st.kind = kDrawNone;
                store_state(a.dstate + b, st);
            }
        }
        return;
    }
    if (sampling) {  // target probability of every node's token under its parent's row
        for (int c = 1 + tid; c < N; c += kBlock) {
            const int pp = ts.par[c];
            const double l = (double)Ld<T>::one(logits + ((size_t)b * N + pp) * V + ts.tok[c]);
            ts.pc[c] = exp((l - (double)ts.M[pp]) / Td) / ts.Z[pp];
        }
        __syncthreads();
    }

    int cur = 0, d = 0, nexcl = 0;
    for (;;) {
        if (ts.M[cur] == -INFINITY) {  // a row the walk reaches has no finite logit
            bad = true;
            break;
        }
        // children of cur in ascending node id (ordered compaction)
        int count = 0;
        for (int base = cur + 1; base < N; base += kBlock) {
            const int c = base + tid;
            const bool f = c < N && ts.par[c] == cur;
            const unsigned long long m = __ballot(f);
            if (lane == 0) ts.wcnt[wave] = __popcll(m);
            __syncthreads();
            int off = count, total = 0;
            for (int w = 0; w < kWaves; ++w) {
                if (w < wave) off += ts.wcnt[w];
                total += ts.wcnt[w];
            }
            if (f) ts.kids[off + __popcll(m & ((1ull << lane) - 1ull))] = c;
            __syncthreads();
            count += total;
        }
        if (count == 0) {
            nexcl = 0;
            break;
        }
        if (tid == 0) {
            int ch = -1;
            if (sampling) {
                const double u = (double)a.coins[(size_t)b * (D + 1) + d];
                const double tha = (double)a.th_acc, ths = (double)a.th_single;
                double acc = 0.0;
                for (int j = 0; j < count; ++j) {
                    const double pc = ts.pc[ts.kids[j]];
                    acc += pc;
                    if (u <= acc / tha || pc >= ths) {
                        ch = j;
                        break;
                    }
                }
            } else {
                for (int j = 0; j < count; ++j)
                    if (ts.tok[ts.kids[j]] == ts.arg[cur]) {
                        ch = j;
                        break;
                    }
            }
            ts.chosen = ch;
        }
        __syncthreads();
        const int ch = ts.chosen;
        if (ch < 0) {
            nexcl = sampling ? count : 0;
            for (int j = tid; j < nexcl; j += kBlock) ts.excl[j] = ts.tok[ts.kids[j]];
            __syncthreads();
            break;
        }
        const int c = ts.kids[ch];
        if (tid == 0) {
            out[d] = ts.tok[c];
            nodes[d] = c;
            if (probs) probs[d] = sampling ? (float)ts.pc[c] : 0.f;
        }
        __syncthreads();
        cur = c;
        ++d;
    }

    if (bad) {  // reached a row with no finite logit: nothing of the walk is kept
        __syncthreads();
        for (int e = tid; e <= D; e += kBlock) {
            out[e] = -1;
            if (e < D) nodes[e] = -1;
            if (probs) probs[e] = 0.f;
        }
        if (tid == 0) {
            a.accept_len[b] = -1;
            if (sampling) {
                DrawState st = {};
                st.kind = kDrawNone;
                store_state(a.dstate + b, st);
            }
        }
        return;
    }
    // the last token: greedy emits the argmax of row cur; sampling hands row cur and the
    // distinct tokens of the children tried last to the final draw
    if (sampling) {
        int32_t* ex = a.excl + (size_t)b * SPEC_MAX_N;
        for (int j = tid; j < nexcl; j += kBlock) {  // keep the first copy of each token
            const int t = ts.excl[j];
            bool dup = false;
            for (int i = 0; i < j && !dup; ++i) dup = ts.excl[i] == t;
            ts.kids[j] = dup ? -1 : t;
        }
        __syncthreads();
        if (tid == 0) {
            int n = 0;
            for (int j = 0; j < nexcl; ++j)
                if (ts.kids[j] >= 0) ex[n++] = ts.kids[j];
            DrawState st = {};
            st.kind = kDrawTarget;
            st.row = b * N + cur;
            st.out = b * (D + 1) + d;
            st.coin = b * (D + 1) + D;
            st.nexcl = n;
            st.M = ts.M[cur];
            st.Z = ts.Z[cur];
            st.invZ = (float)(1.0 / ts.Z[cur]);
            st.T = Td;
            store_state(a.dstate + b, st);
        }
    } else if (tid == 0) {
        out[d] = ts.arg[cur];
        if (probs) probs[d] = 0.f;
    }
    if (tid == 0) a.accept_len[b] = d;
    for (int e = d + 1 + tid; e <= D; e += kBlock) {
        out[e] = -1;
        if (probs) probs[e] = 0.f;
    }
    for (int e = d + tid; e < D; e += kBlock) nodes[e] = -1;
}

// ---------------------------------------------------------------------------------------
// The cluster hand-off used by the walks (k_greedy_walk, k_chain_walk, k_tree_walk,
// k_mss_walk): W workgroups share one request, each owning a slice of every row, and
// after every pass they exchange three 32-bit payloads per workgroup.

constexpr int kMaxCluster = 16;    // workgroups sharing one request's walk
constexpr int kSpinMax = 1 << 18;  // default bound of a cluster wait (never reached when all run)

struct XSmem {
    uint32_t xp[kMaxCluster][3];  // payloads of a cluster step, by workgroup
    int xbad;
};

// The tag of a call's hand-off words comes from a counter in the workspace header
// (hdr[0]); hdr[1] counts the requests whose workgroups have all finished, and word
// kExitBase + b is request b's exit word.  Every workgroup reads the counter when it
// starts, and the counter advances only when every workgroup of the call has finished:
// each workgroup counts itself out of its request's exit word, the last one out of a
// request reports the request, and the last report advances the counter.  No workgroup
// can therefore read a later value than the one its call started with, whenever it
// starts, so all of a call's hand-offs carry one tag and the next call on the stream
// carries the next one: the tag changes from call to call with no host state, and a
// captured graph replays correctly.  The header must be zero before the first call;
// every exit word is reset by the last workgroup out of its request, so the header is
// zero again (except hdr[0]) between calls, whatever the shapes of the calls.
//
// The exit word also carries the request's result.  Bits 0-5 count the workgroups out,
// bits 6-11 those whose hand-off wait ran out, and bits 12-31 hold workgroup 0's result
// plus 2 (accept_len, or -1 for an invalid request).  The last workgroup out writes
// accept_len: workgroup 0's result, or SPEC_ROW_RETRY when any member gave up, since a
// member that gave up may have left its part of the request undone (its slice's final
// weights, or the final token) even where workgroup 0 saw every word it waited for.
//
// Only wave 0 reads the counter (thread 0 publishes, lanes below W wait), and nothing
// waits for the read until the first hand-off, so it overlaps the first row pass.
constexpr int kExitBase = 64;      // first exit word (byte 256 of the header)
constexpr int kExitWords = 4096;   // requests per call that a walk with W > 1 can take

__device__ inline uint32_t walk_epoch(const unsigned* hdr) {
    return (hdr && threadIdx.x < 64)
               ? __hip_atomic_load(hdr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : 0u;
}
__device__ inline uint32_t walk_tag(uint32_t epoch) {
    return epoch % 0xffffffffu + 1u;  // never 0, the value zeroed slots hold
}

// Called once by every workgroup of a walk, after its last hand-off and its share of the
// outputs.  `result` is workgroup 0's accept_len (-1: invalid request); `gaveup` is true
// when one of this workgroup's waits ran out.  Without hand-off words (W = 1, hdr null)
// workgroup 0 writes accept_len itself.
__device__ inline void walk_end(unsigned* hdr, uint32_t epoch, int b, int w, int W,
                                bool gaveup, int result, int32_t* accept_len) {
    if (threadIdx.x != 0) return;
    if (!hdr) {
        if (w == 0) accept_len[b] = gaveup ? SPEC_ROW_RETRY : result;
        return;
    }
    const unsigned inc = 1u | (gaveup ? 1u << 6 : 0u) |
                         (w == 0 ? (unsigned)(result + 2) << 12 : 0u);
    unsigned* ex = hdr + kExitBase + b;
    const unsigned now =
        __hip_atomic_fetch_add(ex, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + inc;
    if ((int)(now & 63u) != W) return;  // not the last workgroup of the request out
    __hip_atomic_store(ex, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    accept_len[b] = ((now >> 6) & 63u) ? SPEC_ROW_RETRY : (int)(now >> 12) - 2;
    const unsigned done = __hip_atomic_fetch_add(hdr + 1, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x / W - 1) {  // the call's last request
        __hip_atomic_store(hdr + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(hdr, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One step of a cluster: every workgroup of the request hands three 32-bit payloads to
// the others.  Each payload travels in a 64-bit word whose high half is the call's tag;
// words are written and read whole with agent-scope atomics, which are coherent across
// the XCDs, so a reader that sees the tag sees the payload and no fence is needed.  Slot
// (step, workgroup) is written once per call.  The wait is bounded (`spin` polls): if a
// word never arrives, the step fails, and the request reports SPEC_ROW_RETRY instead of
// hanging.  With W = 1 the payloads stay in LDS.
__device__ void cluster_publish(unsigned long long* slots, int step, int W, int w,
                                uint32_t tag, uint32_t p0, uint32_t p1, uint32_t p2,
                                XSmem& sm) {
    if (threadIdx.x != 0) return;
    if (W == 1) {  // nothing to hand over: the payloads stay in LDS
        sm.xp[0][0] = p0;
        sm.xp[0][1] = p1;
        sm.xp[0][2] = p2;
        return;
    }
    unsigned long long* base = slots + (size_t)step * W * 3;
    const unsigned long long t = (unsigned long long)tag << 32;
    __hip_atomic_store(base + w * 3 + 0, t | p0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(base + w * 3 + 1, t | p1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(base + w * 3 + 2, t | p2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits for the W payloads of `step` (sm.xp[w][0..2] afterwards, in every thread).
__device__ bool cluster_wait(unsigned long long* slots, int step, int W, uint32_t tag,
                             int spin_max, XSmem& sm) {
    const int tid = threadIdx.x;
    if (W == 1) {
        __syncthreads();
        return true;
    }
    if (tid == 0) sm.xbad = 0;
    __syncthreads();
    if (tid < W) {
        unsigned long long* q = slots + (size_t)step * W * 3 + tid * 3;
        unsigned long long v0 = 0, v1 = 0, v2 = 0;
        for (int spin = 1;; ++spin) {
            v0 = __hip_atomic_load(q + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v1 = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v2 = __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(v0 >> 32) == tag && (uint32_t)(v1 >> 32) == tag &&
                (uint32_t)(v2 >> 32) == tag)
                break;
            if (spin >= spin_max) {
                sm.xbad = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        sm.xp[tid][0] = (uint32_t)v0;
        sm.xp[tid][1] = (uint32_t)v1;
        sm.xp[tid][2] = (uint32_t)v2;
    }
    __syncthreads();
    return sm.xbad == 0;
}

// Publish then wait (a step with nothing to overlap).
__device__ bool cluster_step(unsigned long long* slots, int step, int W, int w, uint32_t tag,
                             int spin_max, uint32_t p0, uint32_t p1, uint32_t p2, XSmem& sm) {
    cluster_publish(slots, step, W, w, tag, p0, p1, p2, sm);
    return cluster_wait(slots, step, W, tag, spin_max, sm);
}

__device__ inline uint32_t dbl_hi(double x) { return (uint32_t)((unsigned long long)__double_as_longlong(x) >> 32); }
__device__ inline uint32_t dbl_lo(double x) { return (uint32_t)__double_as_longlong(x); }
__device__ inline double dbl_of(uint32_t hi, uint32_t lo) {
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Lane j's value of v, in every lane of the wave (j the same in all lanes).
__device__ inline double lane_dbl(double v, int j) {
    return dbl_of((uint32_t)__builtin_amdgcn_readlane((int)dbl_hi(v), j),
                  (uint32_t)__builtin_amdgcn_readlane((int)dbl_lo(v), j));
}

// A row's normaliser from its slices' (max, sum) records after a cluster step (xp[j][0]
// the max, xp[j][1..2] the fp64 sum of exp2((l - max) * s2)): the sum over members j, in
// member order, of z_j exp2((m_j - M) * s2).  Lane j of each wave evaluates member j's
// term, so the W exponentials run side by side instead of one after another; every lane
// then adds the terms in the same order, so all threads of all members hold the same bits.
// The exponential is the row passes' own fp32 one: each z_j is a sum of such
// exponentials, so an fp64 one here would add latency, not accuracy.
__device__ inline double cluster_norm(const XSmem& xs, int W, float M, double Td) {
    const int lane = threadIdx.x & 63;
    const float s2 = kLog2e / (float)Td;
    double term = 0.0;
    if (lane < W) {
        const float mj = __uint_as_float(xs.xp[lane][0]);
        if (mj != -INFINITY)
            term = dbl_of(xs.xp[lane][1], xs.xp[lane][2]) * (double)ex2((mj - M) * s2);
    }
    double Z = 0.0;
    for (int j = 0; j < W; ++j) Z += lane_dbl(term, j);
    return Z;
}

// k_greedy_walk: greedy chain verify position by position, one cluster of W workgroups
// per request (blockIdx = b * W + w, workgroup w owning a slice of whole fine chunks of
// every row).  Each position's slice argmax travels through the cluster hand-off; the
// walk stops at the first mismatch, so rows after it are never read.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_greedy_walk(KArgs a, int W, int per, unsigned* hdr,
                                                        unsigned long long* xslots, int xstride) {
    __shared__ RowSmem rs;
    __shared__ XSmem xs;
    const int tid = threadIdx.x;
    const int b = blockIdx.x / W, w = blockIdx.x - b * W;
    const int R = a.R, G = R - 1, V = a.V;
    const int lo = (int)min((long)V, (long)w * per), hi = (int)min((long)V, (long)lo + per);
    unsigned long long* slots = xslots ? xslots + (size_t)b * xstride : nullptr;
    if (!slots) hdr = nullptr;  // no hand-off words, no tag
    const uint32_t epoch = walk_epoch(hdr), tag = walk_tag(epoch);
    const T* logits = reinterpret_cast<const T*>(a.logits);
    const int32_t* x = a.tokens + (size_t)b * G;
    // lane l of every wave holds draft token l (read once, while the first row streams)
    const int px = (tid & 63) < G ? x[tid & 63] : -1;
    int k = G, last = -1;
    bool bad = false, gaveup = false;
    auto pass = [&](int r) {
        const Part cur = chunk_record<T, false, true, kWalkUnroll>(
            logits + ((size_t)b * R + r) * V, lo, hi, 0.f, rs);
        cluster_publish(slots, r, W, w, tag, __float_as_uint(cur.m), (uint32_t)cur.idx, 0u, xs);
    };
    pass(0);
    for (int i = 0; i <= G; ++i) {
        if (!cluster_wait(slots, i, W, tag, a.spin, xs)) {
            bad = gaveup = true;
            break;
        }
        float M = -INFINITY;
        int idx = INT_MAX;
        for (int j = 0; j < W; ++j) {  // slices in order: the lowest index among equal maxima
            const float mj = __uint_as_float(xs.xp[j][0]);
            if (mj > M) {
                M = mj;
                idx = (int)xs.xp[j][1];
            }
        }
        if (M == -INFINITY) {  // a row the walk reaches has no finite logit
            bad = true;
            break;
        }
        last = idx;
        if (i == G) break;
        const int xi = __shfl(px, i);
        if (xi < 0 || xi >= V) {
            bad = true;
            break;
        }
        if (xi != idx) {
            k = i;
            break;
        }
        // a request that walks on is more likely to be among the last to finish: its
        // waves issue ahead of those of requests at earlier positions on the same CU
        if (i == 0)
            __builtin_amdgcn_s_setprio(1);
        else if (i == 1)
            __builtin_amdgcn_s_setprio(2);
        else
            __builtin_amdgcn_s_setprio(3);
        pass(i + 1);
    }
    if (w == 0) {  // workgroup 0 of the cluster writes the request's tokens
        int32_t* out = a.out_tokens + (size_t)b * R;
        for (int e = tid; e < R; e += kBlock)
            out[e] = bad ? -1 : (e < k ? x[e] : (e == k ? last : -1));
    }
    walk_end(hdr, epoch, b, w, W, gaveup, bad ? -1 : k, a.accept_len);
}


// ---------------------------------------------------------------------------------------
// the final draw: k_mass weighs each fine chunk (kFine elements) of the row the token is
// drawn from, and each of its kSegs segments of kSeg elements; k_draw locates the chunk,
// then the segment, then the token (inverse CDF in ascending token id)
//
// Weights, computed identically in both kernels (fp32, no contraction):
//   p_j = exp2((l_j - M) * log2(e) / T) * (1/Z)
//   residual (chain, rejected at k):   w_j = max(0, p_j - q_j)
//   residual (tree with draft rows):   w_j = max(0, p_j - c * q_j), c from the walk
//   target (chain bonus, tree):        w_j = p_j, with the excluded tokens at 0 (tree)
// Fallback when the total weight is not positive: w_j = p_j (the plain target row).
// Segment and chunk sums are fp64 sums of fp32 sums of four weights.

// Order-preserving integer key of a float: a < b iff key(a) < key(b), and a == b iff
// key(a) == key(b) (NaN aside; -0.0 and +0.0 share the key of +0.0, as they compare
// equal).  A bf16 value widened to fp32 has the same order through its top 16 key bits.
__device__ inline uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);  // -0.0 + 0.0 is +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Parameters of the draw weights of one request.
struct WParams {
    float M, s2, invZ;  // target row
    float cq;           // residual coefficient on the draft row
    uint32_t thp;       // filtered: target tokens with a key below thp weigh 0
    float Mq, invZq;    // draft logits row (kQ == 2)
    uint32_t thq;
};

// kQ: 0 = no draft row (target weights), 1 = draft probabilities (fp32), 2 = draft logits
// (same dtype as the target, filtered by thq).  kFilt: the target row is filtered by thp.
template <typename T, int kQ>
struct QRow {
    typedef u32x4 Raw;  // four fp32 probabilities (or unused)
};
template <typename T>
struct QRow<T, 2> {
    typedef typename Quad<T>::Raw Raw;
};

template <typename T, int kQ, bool kFilt>
__device__ inline float draw_weight(const T* row, const void* q, int j, const WParams& W,
                                    float& p) {
    const float l = Ld<T>::one(row + j);
    p = ex2((l - W.M) * W.s2) * W.invZ;
    if (kFilt && order_key(l) < W.thp) p = 0.f;
    if (kQ == 0) return p;
    float qv;
    if (kQ == 1) {
        qv = static_cast<const float*>(q)[j];
    } else {
        const float d = Ld<T>::one(static_cast<const T*>(q) + j);
        qv = ex2((d - W.Mq) * W.s2) * W.invZq;
        if (order_key(d) < W.thq) qv = 0.f;
    }
    return fmaxf(p - W.cq * qv, 0.f);
}

// Weights of four consecutive elements: `pw` gets the sum of the plain (filtered) p_j,
// `ww` the sum of the draw weights.
template <typename T, int kQ, bool kFilt>
__device__ inline void weigh4(const typename Quad<T>::Raw& lr, const typename QRow<T, kQ>::Raw& qr,
                              const WParams& W, float& pw, float& ww) {
    float l[4];
    Quad<T>::unpack(lr, l);
    if (kFilt) {  // every target weight filtered out: both sums are +0, no exponential needed
        bool kept = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) kept = kept || order_key(l[e]) >= W.thp;
        if (!kept) {
            pw = 0.f;
            ww = 0.f;
            return;
        }
    }
    float qv[4] = {0.f, 0.f, 0.f, 0.f};
    if (kQ == 1) {
        const u32x4& r = reinterpret_cast<const u32x4&>(qr);
        qv[0] = __uint_as_float(r.x);
        qv[1] = __uint_as_float(r.y);
        qv[2] = __uint_as_float(r.z);
        qv[3] = __uint_as_float(r.w);
    } else if (kQ == 2) {
        float d[4];
        Quad<T>::unpack(reinterpret_cast<const typename Quad<T>::Raw&>(qr), d);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[e] = ex2((d[e] - W.Mq) * W.s2) * W.invZq;
            if (order_key(d[e]) < W.thq) qv[e] = 0.f;
        }
    }
    float ps = 0.f, ws = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float p = ex2((l[e] - W.M) * W.s2) * W.invZ;
        if (kFilt && order_key(l[e]) < W.thp) p = 0.f;
        ps += p;
        if (kQ != 0) ws += fmaxf(p - W.cq * qv[e], 0.f);
    }
    pw = ps;
    ww = kQ != 0 ? ws : ps;
}

// LDS slot of quad q (0..1023) of a fine chunk in the weight staging arrays: the 16 quads of
// segment g (q = 16 g + i) sit in column g of a 16 x 65 array, so the lane summing segment g
// reads consecutive words across lanes (no bank conflicts; rows padded to 65 so that the
// writers, 16 consecutive lanes per row, spread over the banks too).
constexpr int kStageRow = 65;
static_assert(kSegs == 64 && kFine / 4 == 16 * kSegs, "a chunk is 1024 quads in 64 segments of 16");
__device__ inline int stage_slot(int q) { return (q & 15) * kStageRow + (q >> 4); }

template <typename V>
__device__ inline V ld_stream_any(const V* p) {
    return __builtin_nontemporal_load(p);
}

// Lane t of the block takes elements 4t..4t+3 of each 1024-element quarter u of the chunk
// (quad q = u * kBlock + t) and leaves their weight sums in slot stage_slot(q) of `pw` /
// `ww` (LDS): segment g is quads 16g .. 16g + 15.
template <typename T, int kQ, bool kFilt>
__device__ inline void chunk_weights(const T* rowp, const void* qrow, int n, bool fast,
                                     const WParams& W, float* pw, float* ww) {
    const int tid = threadIdx.x;
    typedef typename QRow<T, kQ>::Raw QR;
    if (fast) {  // full, 16-byte aligned chunk: every load in flight at once
        const Quad<T>* lq = reinterpret_cast<const Quad<T>*>(rowp);
        const QR* qq = static_cast<const QR*>(qrow);
        typename Quad<T>::Raw lr[4];
        QR qr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            lr[u] = lq[u * kBlock + tid].raw;
            if (kQ != 0) qr[u] = ld_stream_any(qq + u * kBlock + tid);
        }
        __builtin_amdgcn_sched_barrier(0);  // all of the chunk's loads before the first use
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float p4, w4;
            weigh4<T, kQ, kFilt>(lr[u], qr[u], W, p4, w4);
            pw[stage_slot(u * kBlock + tid)] = p4;
            ww[stage_slot(u * kBlock + tid)] = w4;
        }
        return;
    }
    for (int u = 0; u < 4; ++u) {
        float p4 = 0.f, w4 = 0.f;
        for (int i = 0; i < 4; ++i) {
            const int e = u * 4 * kBlock + 4 * tid + i;
            if (e < n) {
                float p;
                const float w = draw_weight<T, kQ, kFilt>(rowp, qrow, e, W, p);
                p4 += p;
                w4 += w;
            }
        }
        pw[stage_slot(u * kBlock + tid)] = p4;
        ww[stage_slot(u * kBlock + tid)] = kQ != 0 ? w4 : p4;
    }
}

// One workgroup per chain request: the acceptance scan, its outputs and the draw state.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_chain_accept(KArgs a) {
    __shared__ Smem sm;
    __shared__ RecSmem rs;
    const DrawState st = chain_accept<T>(a, blockIdx.x, true, sm, rs);
    if (threadIdx.x == 0) store_state(a.dstate + blockIdx.x, st);
}

struct MassSmem {
    float pw[16 * kStageRow];  // plain target weight of each quad of a chunk (stage_slot)
    float ww[16 * kStageRow];  // draw weight of the same
};

// Two chunks' staging, weighed together and summed by waves 0 and 1 (the walks).
struct MassSmem2 {
    MassSmem s[2];
};

// Four chunks' staging, summed by the four waves (one chunk each), and a copy of the chunk
// masses of the first kLdsChunks chunks of the slice (the walk's draw reads them there
// instead of reading back what the workgroup has just written to memory).
constexpr int kLdsChunks = 64;
struct MassSmem4 {
    MassSmem s[kWaves];
    double cm[kLdsChunks];   // mass of chunk cb + i
    double cmf[kLdsChunks];  // its plain target weight (the fallback)
};

// The draw weights' parameters and draft row of a request's draw state.
template <typename T, bool kFilt>
__device__ inline WParams draw_params(const KArgs& a, const DrawState& st, const void*& qrow) {
    WParams W;
    W.M = st.M;
    W.s2 = kLog2e / (float)st.T;
    W.invZ = st.invZ;
    W.thp = kFilt ? st.thp : 0u;
    W.Mq = st.Mq;
    W.invZq = st.invZq;
    W.thq = st.thq;
    W.cq = st.cq;
    qrow = nullptr;
    if (st.kind == kDrawResidual)
        qrow = kFilt ? static_cast<const void*>(static_cast<const T*>(a.dlogits) + (size_t)st.qrow * a.V)
                     : static_cast<const void*>(a.q + (size_t)st.qrow * a.V);
    return W;
}

// Tree draws: the rejected children's tokens weigh nothing.  Every quad of fine chunk c
// that holds one of them (ex[0 .. st.nexcl)) is weighed again without them: the other
// elements' weights added in weigh4's order, which gives the bits weigh4 gives with the
// excluded weights at zero.  Its staged draw weight (ms.ww) is replaced; the plain target
// weight (ms.pw, for the fallback) keeps every token.  One wave; two lanes that share a
// quad write the same value.  The caller syncs before the segment sums.
template <typename T, bool kFilt>
__device__ inline void exclude_quads(const KArgs& a, const DrawState& st, const WParams& W,
                                     const T* rowp, int c, MassSmem& ms, const int32_t* ex) {
    const int lane = threadIdx.x & 63;
    const int c0 = c * kFine;
    const int n = min(kFine, a.V - c0);
    for (int e = lane; e < st.nexcl; e += 64) {
        const int t = ex[e];
        if (t < c0 || t >= c0 + n) continue;
        const int q = (t - c0) >> 2;
        float w4 = 0.f;
        for (int i = 0; i < 4; ++i) {
            const int j = c0 + 4 * q + i;
            if (j >= c0 + n) break;
            bool out = false;
            for (int f = 0; f < st.nexcl && !out; ++f) out = ex[f] == j;
            if (!out) {
                float p;
                draw_weight<T, 0, kFilt>(rowp, nullptr, j, W, p);
                w4 += p;
            }
        }
        ms.ww[stage_slot(q)] = w4;
    }
}

// Segment and chunk sums of fine chunk c, whose per-quad weights `chunk_weights` left in
// sm.pw / sm.ww: each segment's weight (and the chunk's) in a.seg / a.mass, the plain
// target weight in a.massfb.  Block-wide.
template <typename T, bool kFilt>
__device__ __attribute__((always_inline)) void mass_reduce(const KArgs& a, const DrawState& st,
                                                           const WParams& W, const T* rowp,
                                                           int b, int c, MassSmem& sm,
                                                           const int32_t* ex) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int S2 = a.S2;
    __syncthreads();  // the staging is complete
    if (st.nexcl > 0) {  // tree: the rejected children's quads, weighed again without them
        if (tid < 64) exclude_quads<T, kFilt>(a, st, W, rowp, c, sm, ex);
        __syncthreads();
    }
    if (tid < kSegs) {  // wave 0: lane g sums segment g in ascending order
        double Wt = 0.0, P = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Wt += (double)sm.ww[i * kStageRow + tid];  // quad 16 * tid + i
            P += (double)sm.pw[i * kStageRow + tid];
        }
        a.seg[((size_t)b * S2 + c) * kSegs + tid] = Wt;
        Wt = wave_sum(Wt);
        P = wave_sum(P);
        if (lane == 0) {
            a.mass[(size_t)b * S2 + c] = Wt;
            a.massfb[(size_t)b * S2 + c] = P;
        }
    }
    __syncthreads();  // LDS is reused by the next chunk
}

// Whether fine chunk c takes chunk_weights' fast path (full and 16-byte aligned).
template <typename T, bool kFilt>
__device__ inline bool chunk_fast(const T* rowp, const void* qrow, int c, int V) {
    const size_t qes = kFilt ? sizeof(T) : sizeof(float);
    const int c0 = c * kFine;
    return V - c0 >= kFine && ((uintptr_t)(rowp + c0)) % (4 * sizeof(T)) == 0 &&
           (!qrow || ((uintptr_t)qrow + c0 * qes) % (4 * qes) == 0);
}

// The draw weights of fine chunk c of the row in `st` (see mass_reduce).  Block-wide.
template <typename T, bool kFilt>
__device__ __attribute__((always_inline)) void mass_chunk(const KArgs& a, const DrawState& st,
                                                          const WParams& W, const T* rowp,
                                                          const void* qrow, int b, int c,
                                                          MassSmem& sm, const int32_t* ex) {
    const int c0 = c * kFine;
    const int n = min(kFine, a.V - c0);
    const size_t qes = kFilt ? sizeof(T) : sizeof(float);
    const bool fast = chunk_fast<T, kFilt>(rowp, qrow, c, a.V);
    constexpr int kQr = kFilt ? 2 : 1;
    if (qrow)
        chunk_weights<T, kQr, kFilt>(rowp + c0, static_cast<const char*>(qrow) + c0 * qes, n, fast,
                                     W, sm.pw, sm.ww);
    else
        chunk_weights<T, 0, kFilt>(rowp + c0, nullptr, n, fast, W, sm.pw, sm.ww);
    mass_reduce<T, kFilt>(a, st, W, rowp, b, c, sm, ex);
}

// Segment and chunk sums of chunks cA (staged in sm.s[0], summed by wave 0) and cB (in
// sm.s[1], wave 1; -1 for none), each exactly as mass_reduce sums one chunk.  Block-wide.
template <typename T, bool kFilt>
__device__ __attribute__((always_inline)) void mass_reduce_pair(const KArgs& a,
                                                                const DrawState& st,
                                                                const WParams& W, const T* rowp,
                                                                int b, int cA, int cB,
                                                                MassSmem2& sm,
                                                                const int32_t* ex) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int S2 = a.S2;
    const int c = wv == 0 ? cA : (wv == 1 ? cB : -1);  // the chunk this wave sums
    MassSmem& ms = sm.s[wv & 1];
    __syncthreads();  // the staging is complete
    if (st.nexcl > 0) {  // tree: the rejected children's quads, weighed again without them
        if (c >= 0) exclude_quads<T, kFilt>(a, st, W, rowp, c, ms, ex);
        __syncthreads();
    }
    if (c >= 0) {  // lane g sums segment g in ascending order
        double Wt = 0.0, P = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Wt += (double)ms.ww[i * kStageRow + lane];  // quad 16 * lane + i
            P += (double)ms.pw[i * kStageRow + lane];
        }
        a.seg[((size_t)b * S2 + c) * kSegs + lane] = Wt;
        Wt = wave_sum(Wt);
        P = wave_sum(P);
        if (lane == 0) {
            a.mass[(size_t)b * S2 + c] = Wt;
            a.massfb[(size_t)b * S2 + c] = P;
        }
    }
    __syncthreads();  // the staging is reused by the next pair
}

// The draw weights of fine chunks [cb, ce) of the row in `st`, as mass_chunk computes
// them chunk by chunk, with the loads of chunk c + 1 in flight while chunk c's segment
// sums are formed: a chunk's registers are free once its weights are in LDS.  Block-wide.
template <typename T, int kQ, bool kFilt>
__device__ __attribute__((always_inline)) void mass_slice_q(const KArgs& a, const DrawState& st,
                                                            const WParams& W, const T* rowp,
                                                            const void* qrow, int b, int cb,
                                                            int ce, MassSmem& sm,
                                                            const int32_t* ex) {
    typedef typename Quad<T>::Raw LR;
    typedef typename QRow<T, kQ>::Raw QR;
    const int tid = threadIdx.x;
    const size_t qes = kFilt ? sizeof(T) : sizeof(float);
    LR lr[4];
    QR qr[4];
    auto load = [&](int c) {
        const Quad<T>* lq = reinterpret_cast<const Quad<T>*>(rowp + c * kFine);
        const QR* qq = kQ != 0 ? reinterpret_cast<const QR*>(static_cast<const char*>(qrow) +
                                                             (size_t)c * kFine * qes)
                               : nullptr;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            lr[u] = lq[u * kBlock + tid].raw;
            if (kQ != 0) qr[u] = ld_stream_any(qq + u * kBlock + tid);
        }
    };
    bool fast = cb < ce && chunk_fast<T, kFilt>(rowp, qrow, cb, a.V);
    if (fast) load(cb);
    for (int c = cb; c < ce; ++c) {
        if (fast) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float p4, w4;
                weigh4<T, kQ, kFilt>(lr[u], qr[u], W, p4, w4);
                sm.pw[stage_slot(u * kBlock + tid)] = p4;
                sm.ww[stage_slot(u * kBlock + tid)] = w4;
            }
        } else {
            const int c0 = c * kFine;
            chunk_weights<T, kQ, kFilt>(rowp + c0,
                                        kQ != 0 ? static_cast<const char*>(qrow) + c0 * qes : nullptr,
                                        min(kFine, a.V - c0), false, W, sm.pw, sm.ww);
        }
        fast = c + 1 < ce && chunk_fast<T, kFilt>(rowp, qrow, c + 1, a.V);
        if (fast) load(c + 1);
        __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads before this one's sums
        mass_reduce<T, kFilt>(a, st, W, rowp, b, c, sm, ex);
    }
}

template <typename T, bool kFilt>
__device__ __attribute__((always_inline)) void mass_slice(const KArgs& a, const DrawState& st,
                                                          const WParams& W, const T* rowp,
                                                          const void* qrow, int b, int cb, int ce,
                                                          MassSmem& sm, const int32_t* ex) {
    if (qrow)
        mass_slice_q<T, kFilt ? 2 : 1, kFilt>(a, st, W, rowp, qrow, b, cb, ce, sm, ex);
    else
        mass_slice_q<T, 0, kFilt>(a, st, W, rowp, nullptr, b, cb, ce, sm, ex);
}

// The draw weights of fine chunks [cb, ce) of the row in `st`, as mass_chunk computes them,
// two chunks per round: both chunks' loads are in flight together, and waves 0 and 1 sum
// one chunk each.  Block-wide.
template <typename T, int kQ, bool kFilt>
__device__ __attribute__((always_inline)) void mass_slice2_q(const KArgs& a, const DrawState& st,
                                                            const WParams& W, const T* rowp,
                                                            const void* qrow, int b, int cb,
                                                            int ce, MassSmem2& sm,
                                                            const int32_t* ex) {
    typedef typename Quad<T>::Raw LR;
    typedef typename QRow<T, kQ>::Raw QR;
    const int tid = threadIdx.x;
    const size_t qes = kFilt ? sizeof(T) : sizeof(float);
    LR la[4], lb[4];
    QR qa[4], qb[4];
    auto load = [&](int c, LR* lr, QR* qr) {
        const Quad<T>* lq = reinterpret_cast<const Quad<T>*>(rowp + c * kFine);
        const QR* qq = kQ != 0 ? reinterpret_cast<const QR*>(static_cast<const char*>(qrow) +
                                                             (size_t)c * kFine * qes)
                               : nullptr;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            lr[u] = lq[u * kBlock + tid].raw;
            if (kQ != 0) qr[u] = ld_stream_any(qq + u * kBlock + tid);
        }
    };
    auto stage = [&](int c, bool fast, const LR* lr, const QR* qr, MassSmem& ms) {
        if (fast) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float p4, w4;
                weigh4<T, kQ, kFilt>(lr[u], qr[u], W, p4, w4);
                ms.pw[stage_slot(u * kBlock + tid)] = p4;
                ms.ww[stage_slot(u * kBlock + tid)] = w4;
            }
        } else {
            const int c0 = c * kFine;
            chunk_weights<T, kQ, kFilt>(rowp + c0,
                                        kQ != 0 ? static_cast<const char*>(qrow) + c0 * qes : nullptr,
                                        min(kFine, a.V - c0), false, W, ms.pw, ms.ww);
        }
    };
    for (int c = cb; c < ce; c += 2) {
        const bool two = c + 1 < ce;
        const bool fa = chunk_fast<T, kFilt>(rowp, qrow, c, a.V);
        const bool fb = two && chunk_fast<T, kFilt>(rowp, qrow, c + 1, a.V);
        if (fa) load(c, la, qa);
        if (fb) load(c + 1, lb, qb);
        __builtin_amdgcn_sched_barrier(0);  // both chunks' loads before the first use
        stage(c, fa, la, qa, sm.s[0]);
        if (two) stage(c + 1, fb, lb, qb, sm.s[1]);
        mass_reduce_pair<T, kFilt>(a, st, W, rowp, b, c, two ? c + 1 : -1, sm, ex);
    }
}

template <typename T, bool kFilt>
__device__ __attribute__((always_inline)) void mass_slice2(const KArgs& a, const DrawState& st,
                                                          const WParams& W, const T* rowp,
                                                          const void* qrow, int b, int cb, int ce,
                                                          MassSmem2& sm, const int32_t* ex) {
    if (qrow)
        mass_slice2_q<T, kFilt ? 2 : 1, kFilt>(a, st, W, rowp, qrow, b, cb, ce, sm, ex);
    else
        mass_slice2_q<T, 0, kFilt>(a, st, W, rowp, nullptr, b, cb, ce, sm, ex);
}

// Segment and chunk sums of chunks c0 .. cend - 1 (at most kWaves), chunk c0 + w staged in
// sm.s[w] and summed by wave w exactly as mass_reduce sums one chunk.  Block-wide.
template <typename T, bool kFilt>
__device__ __attribute__((always_inline)) void mass_reduce_quad(const KArgs& a,
                                                                const DrawState& st,
                                                                const WParams& W, const T* rowp,
                                                                int b, int c0, int cend,
                                                                MassSmem4& sm,
                                                                const int32_t* ex, int cb) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int S2 = a.S2;
    const int c = c0 + wv < cend ? c0 + wv : -1;  // the chunk this wave sums
    MassSmem& ms = sm.s[wv];
    __syncthreads();  // the staging is complete
    if (st.nexcl > 0) {  // tree: the rejected children's quads, weighed again without them
        if (c >= 0) exclude_quads<T, kFilt>(a, st, W, rowp, c, ms, ex);
        __syncthreads();
    }
    if (c >= 0) {  // lane g sums segment g in ascending order
        double Wt = 0.0, P = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Wt += (double)ms.ww[i * kStageRow + lane];  // quad 16 * lane + i
            P += (double)ms.pw[i * kStageRow + lane];
        }
        a.seg[((size_t)b * S2 + c) * kSegs + lane] = Wt;
        Wt = wave_sum(Wt);
        P = wave_sum(P);
        if (lane == 0) {
            a.mass[(size_t)b * S2 + c] = Wt;
            a.massfb[(size_t)b * S2 + c] = P;
            if (c - cb < kLdsChunks) {
                sm.cm[c - cb] = Wt;
                sm.cmf[c - cb] = P;
            }
        }
    }
    __syncthreads();  // the staging is reused by the next four chunks (and cm is complete)
}

// The draw weights of fine chunks [cb, ce) of the row in `st`, as mass_chunk computes them:
// chunks are weighed one after another into four LDS stagings, and every four chunks the
// four waves sum one chunk each, so the barriers and the sums are paid once per four
// chunks instead of once per chunk.  Block-wide.
//
// stop_at >= 0: stop after the first group of four chunks with which the chunk masses,
// added in chunk order, reach stop_at; returns the end of the chunks weighed.
template <typename T, int kQ, bool kFilt>
__device__ __attribute__((always_inline)) int mass_slice4_q(const KArgs& a, const DrawState& st,
                                                            const WParams& W, const T* rowp,
                                                            const void* qrow, int b, int cb,
                                                            int ce, MassSmem4& sm,
                                                            const int32_t* ex,
                                                            double stop_at = -1.0) {
    typedef typename Quad<T>::Raw LR;
    typedef typename QRow<T, kQ>::Raw QR;
    const int tid = threadIdx.x;
    const size_t qes = kFilt ? sizeof(T) : sizeof(float);
    LR la[4];
    QR qa[4];
    auto load = [&](int c, LR* lr, QR* qr) {
        const Quad<T>* lq = reinterpret_cast<const Quad<T>*>(rowp + c * kFine);
        const QR* qq = kQ != 0 ? reinterpret_cast<const QR*>(static_cast<const char*>(qrow) +
                                                             (size_t)c * kFine * qes)
                               : nullptr;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            lr[u] = lq[u * kBlock + tid].raw;
            if (kQ != 0) qr[u] = ld_stream_any(qq + u * kBlock + tid);
        }
    };
    auto stage = [&](int c, bool fast, const LR* lr, const QR* qr, MassSmem& ms) {
        if (fast) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float p4, w4;
                weigh4<T, kQ, kFilt>(lr[u], qr[u], W, p4, w4);
                ms.pw[stage_slot(u * kBlock + tid)] = p4;
                ms.ww[stage_slot(u * kBlock + tid)] = w4;
            }
        } else {
            const int c0 = c * kFine;
            chunk_weights<T, kQ, kFilt>(rowp + c0,
                                        kQ != 0 ? static_cast<const char*>(qrow) + c0 * qes : nullptr,
                                        min(kFine, a.V - c0), false, W, ms.pw, ms.ww);
        }
    };
    for (int c0 = cb; c0 < ce; c0 += kWaves) {
#pragma unroll
        for (int j = 0; j < kWaves; ++j) {
            const int c = c0 + j;
            if (c < ce) {
                const bool f = chunk_fast<T, kFilt>(rowp, qrow, c, a.V);
                if (f) load(c, la, qa);
                __builtin_amdgcn_sched_barrier(0);
                stage(c, f, la, qa, sm.s[j]);
            }
        }
        const int c1 = min(ce, c0 + kWaves);
        mass_reduce_quad<T, kFilt>(a, st, W, rowp, b, c0, c1, sm, ex, cb);
        if (stop_at >= 0.0) {  // the masses were written before the reduction's last barrier
            double cum = 0.0;
            for (int c = cb; c < c1; ++c)
                cum += c - cb < kLdsChunks ? sm.cm[c - cb] : a.mass[(size_t)b * a.S2 + c];
            if (cum >= stop_at) return c1;
        }
    }
    return ce;
}

template <typename T, bool kFilt>
__device__ __attribute__((always_inline)) int mass_slice4(const KArgs& a, const DrawState& st,
                                                          const WParams& W, const T* rowp,
                                                          const void* qrow, int b, int cb, int ce,
                                                          MassSmem4& sm, const int32_t* ex,
                                                          double stop_at = -1.0) {
    if (qrow)
        return mass_slice4_q<T, kFilt ? 2 : 1, kFilt>(a, st, W, rowp, qrow, b, cb, ce, sm, ex,
                                                      stop_at);
    return mass_slice4_q<T, 0, kFilt>(a, st, W, rowp, nullptr, b, cb, ce, sm, ex, stop_at);
}

// One workgroup per (request, fine chunk).
template <typename T, bool kFilt>
__global__ __launch_bounds__(kBlock) void k_mass(KArgs a) {
    __shared__ MassSmem sm;
    const int S2 = a.S2;
    const int b = blockIdx.x / S2;
    const int c = blockIdx.x - b * S2;
    const DrawState st = load_state(a.dstate + b);
    if (st.kind == kDrawNone) return;
    const T* rowp = reinterpret_cast<const T*>(a.logits) + (size_t)st.row * a.V;
    const void* qrow;
    const WParams W = draw_params<T, kFilt>(a, st, qrow);
    mass_chunk<T, kFilt>(a, st, W, rowp, qrow, b, c, sm,
                         st.nexcl > 0 ? a.excl + (size_t)b * SPEC_MAX_N : nullptr);
}

// Result of a wave-wide search over 64 weights (one per lane).
struct Found {
    int hit;          // first lane with x > 0 whose inclusive prefix reaches t, or -1
    double before;    // weight ahead of `hit`
    int last;         // last lane with x > 0, or -1
    double last_before;
    double total;     // sum of the 64 weights
};

// Among the 64 lanes' values x, counting `carry` ahead of lane 0: the first lane with
// x > 0 whose inclusive prefix reaches t, and the last positive lane (for when rounding
// leaves t beyond the total).  Every lane gets the same result.
__device__ __attribute__((always_inline)) Found wave_find(double x, double t, double carry) {
    const int lane = threadIdx.x & 63;
    double incl = x;
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    const double excl = incl - x;
    const unsigned long long hit = __ballot(x > 0.0 && t <= carry + incl);
    const unsigned long long pos = __ballot(x > 0.0);
    Found f;
    f.hit = hit ? __ffsll((long long)hit) - 1 : -1;
    f.last = pos ? 63 - __clzll((long long)pos) : -1;
    const double eh = __shfl(excl, f.hit < 0 ? 0 : f.hit);
    const double el = __shfl(excl, f.last < 0 ? 0 : f.last);
    f.before = carry + eh;
    f.last_before = carry + el;
    f.total = __shfl(incl, 63);
    return f;
}

// First entry i of w[0..n) with w[i] > 0 whose inclusive prefix reaches t; if rounding
// leaves t beyond the total, the last positive entry; -1 if none is positive.  One full
// wave; every lane returns the entry and the weight before it.
__device__ __attribute__((always_inline)) int wave_locate(const double* w, int n, double t,
                                                        double& before) {
    const int lane = threadIdx.x & 63;
    double carry = 0.0, last_before = 0.0;
    int last = -1;
    for (int i0 = 0; i0 < n; i0 += 64) {
        const Found f = wave_find(i0 + lane < n ? w[i0 + lane] : 0.0, t, carry);
        if (f.hit >= 0) {
            before = f.before;
            return i0 + f.hit;
        }
        if (f.last >= 0) {
            last = i0 + f.last;
            last_before = f.last_before;
        }
        carry += f.total;
    }
    before = last_before;
    return last;
}

// The token inside fine chunk c of the row in `st` whose cumulative weight reaches tc
// (measured from the start of the chunk): its segment from the segment weights (stored by
// the chunk's weighing, or, in the fallback, the plain target row summed here), then the
// element.  One full wave (lanes 0..63); y = -1 if nothing is positive.
template <typename T, bool kFilt>
__device__ __attribute__((always_inline)) void draw_in_chunk(const KArgs& a, const DrawState& st,
                                                             const WParams& W, const T* rowp,
                                                             const void* qrow, int b, int c,
                                                             double tc, bool fallback, int& y,
                                                             float& ly) {
    const int lane = threadIdx.x & 63;
    const int S2 = a.S2, V = a.V;
    const bool resid = qrow != nullptr && !fallback;
    // segment weights: stored by k_mass, or (fallback) the plain target row, summed here
    double x;
    if (!fallback) {
        x = a.seg[((size_t)b * S2 + c) * kSegs + lane];
    } else {
        x = 0.0;
        for (int g0 = 0; g0 < kSegs; g0 += 8) {  // eight segments' loads in flight
            float pv[8];
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const int j = c * kFine + (g0 + g) * kSeg + lane;
                float p = 0.f;
                if (j < V) draw_weight<T, 0, kFilt>(rowp, nullptr, j, W, p);
                pv[g] = p;
            }
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const double sg = wave_sum((double)pv[g]);
                if (lane == g0 + g) x = sg;
            }
        }
    }
    const Found fs = wave_find(x, tc, 0.0);
    const int g = fs.hit >= 0 ? fs.hit : fs.last;
    const double bs = fs.hit >= 0 ? fs.before : fs.last_before;
    if (g >= 0) {
        const double tg = tc - bs;
        const int j = c * kFine + g * kSeg + lane;  // kSeg == 64: one element per lane
        float l = 0.f, w = 0.f;
        if (j < V) {
            l = Ld<T>::one(rowp + j);
            float p;
            constexpr int kQr = kFilt ? 2 : 1;
            w = resid ? draw_weight<T, kQr, kFilt>(rowp, qrow, j, W, p)
                      : draw_weight<T, 0, kFilt>(rowp, nullptr, j, W, p);
            if (!fallback && st.nexcl > 0) {
                const int32_t* ex = a.excl + (size_t)b * SPEC_MAX_N;
                for (int e = 0; e < st.nexcl; ++e)
                    if (ex[e] == j) w = 0.f;
            }
        }
        const Found fe = wave_find((double)w, tg, 0.0);
        const int f = fe.hit >= 0 ? fe.hit : fe.last;
        if (f >= 0) {
            y = c * kFine + g * kSeg + f;
            ly = __shfl(l, f);
        }
    }
}

// k_chain_walk: chain rejection sampling position by position, one cluster of W
// workgroups per request (blockIdx = b * W + w, workgroup w owning a slice of whole fine
// chunks of every row).  At each position the slices' (max, normaliser) travel through
// the cluster hand-off and every workgroup takes the same acceptance decision; the walk
// stops at the first rejection (or after the bonus row), so rows after it are never
// read.  Each workgroup then weighs its slice of the row the last token is drawn from
// (the residual against q, or the plain row for the bonus), which k_draw searches.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_chain_walk(KArgs a, int W, int per, unsigned* hdr,
                                                       unsigned long long* xslots, int xstride) {
    __shared__ RowSmem rs;
    __shared__ XSmem xs;
    __shared__ MassSmem4 ms;
    __shared__ float sp[kMaxRows];
    __shared__ int sflag;
    const int tid = threadIdx.x;
    const int b = blockIdx.x / W, w = blockIdx.x - b * W;
    const int R = a.R, G = R - 1, V = a.V;
    const int lo = (int)min((long)V, (long)w * per), hi = (int)min((long)V, (long)lo + per);
    unsigned long long* slots = xslots ? xslots + (size_t)b * xstride : nullptr;
    if (!slots) hdr = nullptr;  // no hand-off words, no tag
    const uint32_t epoch = walk_epoch(hdr), tag = walk_tag(epoch);
    // The walking waves issue ahead of the final-weight waves of requests that have
    // stopped (the priority drops again before the weights): the walks of the longest
    // requests are the call's critical path, the weights of the others are not.
    __builtin_amdgcn_s_setprio(3);
    const T* logits = reinterpret_cast<const T*>(a.logits);
    // Every per-request input is read up front and waited for only where it is used, so
    // the reads overlap the first row pass: the temperature and the final coin (checked
    // after the first hand-off), and in wave 0, lane l's draft token and coin.
    const float Tf = a.temperature[b];
    const float uG = a.coins[(size_t)b * R + G];
    int px = -1;
    float pu = 0.f;
    if (tid < G) {
        px = a.tokens[(size_t)b * G + tid];
        pu = a.coins[(size_t)b * R + tid];
    }
    bool bad = false, gaveup = false;
    const double Td = (double)Tf;
    const float s2 = kLog2e / Tf;
    int k = G;
    float M = -INFINITY;
    double Z = 0.0;
    auto pass = [&](int r) {
        const T* rowp = logits + ((size_t)b * R + r) * V;
        const Part cur =
            a.walk_temporal ? chunk_record<T, true, false, kWalkUnroll>(rowp, lo, hi, s2, rs)
                            : chunk_record<T, true, true, kWalkUnroll>(rowp, lo, hi, s2, rs);
        cluster_publish(slots, r, W, w, tag, __float_as_uint(cur.m), dbl_hi(cur.z), dbl_lo(cur.z),
                        xs);
    };
    pass(0);
    for (int i = 0; i <= G; ++i) {
        const T* rowp = logits + ((size_t)b * R + i) * V;
        int xi = -1;
        float lx = 0.f, qx = 0.f, ui = 0.f;
        if (i < G && tid < 64) {  // the acceptance test's inputs, gathered during the hand-off
            xi = __shfl(px, i);
            ui = __shfl(pu, i);
            if (tid == 0 && xi >= 0 && xi < V) {
                lx = Ld<T>::one(rowp + xi);
                qx = a.q[((size_t)b * G + i) * V + xi];
            }
        }
        if (!cluster_wait(slots, i, W, tag, a.spin, xs)) {
            bad = gaveup = true;
            break;
        }
        if (i == 0 && (!(isfinite(Tf) && Tf > 0.f) || !(uG > 0.f && uG <= 1.f))) {
            bad = true;
            break;
        }
        M = -INFINITY;
        for (int j = 0; j < W; ++j) M = fmaxf(M, __uint_as_float(xs.xp[j][0]));
        Z = cluster_norm(xs, W, M, Td);
        if (M == -INFINITY) {  // a row the walk reaches has no finite logit
            bad = true;
            break;
        }
        if (i == G) break;  // every draft accepted: the bonus from row G
        if (tid == 0) {  // 0 = rejected, 1 = accepted, 2 = unusable input
            int flag;
            if (xi < 0 || xi >= V || !(ui > 0.f && ui <= 1.f) || !(qx >= 0.f && isfinite(qx))) {
                flag = 2;
            } else {
                const double p = (double)ex2((lx - M) * s2) / Z;
                const double q = (double)qx;
                flag = (q > 0.0 ? (p > 0.0 && (double)ui <= p / q) : p > 0.0) ? 1 : 0;
                sp[i] = (float)p;
            }
            sflag = flag;
        }
        __syncthreads();
        const int flag = sflag;
        __syncthreads();
        if (flag == 2) {
            bad = true;
            break;
        }
        if (flag == 0) {
            k = i;
            break;
        }
        pass(i + 1);
    }
    DrawState st = {};
    st.kind = kDrawNone;
    if (!bad) {
        st.kind = k < G ? kDrawResidual : kDrawTarget;
        st.row = b * R + k;
        st.qrow = b * G + k;
        st.out = b * R + k;
        st.coin = b * R + G;
        st.nexcl = 0;
        st.cq = 1.f;
        st.M = M;
        st.Z = Z;
        st.invZ = (float)(1.0 / Z);
        st.T = Td;
        const T* rowp = logits + (size_t)st.row * V;
        const void* qrow;
        const WParams Wp = draw_params<T, false>(a, st, qrow);
        const int cb = lo / kFine, ce = (hi + kFine - 1) / kFine;
        __builtin_amdgcn_s_setprio(0);
        // The bonus draws from the plain target row, whose slice totals the last hand-off
        // already gave: slice j holds z_j exp((m_j - M) / T) / Z of the mass.  Every member
        // finds the owner of u * total from them, and only the owner weighs its slice and
        // draws; the others are done.
        int bonus_owner = -2;  // -2: not taken here
        double bonus_t1 = 0.0;
        if (a.walk_draw && st.kind == kDrawTarget) {
            // A slice holding less than 1e-30 of the mass counts as empty: its weights could
            // underflow in fp32 where the owner weighs them (a slice above it has an element
            // of at least 1e-30 over its at most 64 chunks' 262144 elements, well inside
            // fp32's normal range).
            // Lane j of each wave evaluates slice j's total.
            double mine = 0.0;
            if ((tid & 63) < W) {
                const float mj = __uint_as_float(xs.xp[tid & 63][0]);
                const double tj = mj == -INFINITY ? 0.0
                                                  : dbl_of(xs.xp[tid & 63][1], xs.xp[tid & 63][2]) *
                                                        (double)ex2((mj - M) * s2) / Z;
                mine = tj >= 1e-30 ? tj : 0.0;
            }
            double tot = 0.0;
            for (int j = 0; j < W; ++j) tot += lane_dbl(mine, j);
            const double t = (double)uG * tot;
            double carry = 0.0, before = 0.0, last_before = 0.0;
            int owner = -1, last = -1;
            for (int j = 0; j < W; ++j) {
                const double tj = lane_dbl(mine, j);
                if (tj > 0.0) {
                    if (owner < 0 && t <= carry + tj) {
                        owner = j;
                        before = carry;
                    }
                    last = j;
                    last_before = carry;
                }
                carry += tj;
            }
            if (owner < 0) {  // rounding left u past the total: the last positive slice
                owner = last;
                before = last_before;
            }
            bonus_owner = owner;
            bonus_t1 = t - before;
        }
        int cw = ce;  // end of the chunks weighed
        if (bonus_owner == -2)
            mass_slice4<T, false>(a, st, Wp, rowp, qrow, b, cb, ce, ms, nullptr);
        else if (bonus_owner == w)  // the owner weighs its chunks until they pass its target
            cw = mass_slice4<T, false>(a, st, Wp, rowp, qrow, b, cb, ce, ms, nullptr, bonus_t1);
        if (bonus_owner >= -1) {
            if (w == bonus_owner && tid < 64) {
                const int nc = cw - cb;
                const double mw = tid < nc ? ms.cm[tid] : 0.0;
                const Found f = wave_find(mw, bonus_t1, 0.0);
                const int cl = f.hit >= 0 ? f.hit : f.last;
                const double bc = f.hit >= 0 ? f.before : f.last_before;
                int y = -1;
                float ly = 0.f;
                if (cl >= 0)
                    draw_in_chunk<T, false>(a, st, Wp, rowp, qrow, b, cb + cl, bonus_t1 - bc,
                                            false, y, ly);
                if (tid == 0) {
                    a.out_tokens[st.out] = y;
                    if (a.probs)
                        a.probs[st.out] =
                            y >= 0 ? (float)(exp(((double)ly - (double)st.M) / st.T) / st.Z) : 0.f;
                }
            }
            if (bonus_owner == -1 && w == 0 && tid == 0) {  // no positive weight anywhere
                a.out_tokens[st.out] = -1;
                if (a.probs) a.probs[st.out] = 0.f;
            }
        } else if (a.walk_draw) {
            // The draw, within the cluster (the host sets walk_draw when every slice has at
            // most 64 chunks).  Each member's slice total, as wave 0's scan adds its chunk
            // masses, goes through one more hand-off; the member whose slice holds
            // u * total then locates the chunk, segment and token as k_draw does.  A total
            // that is not positive repeats this with the plain target weights.
            const int nc = ce - cb;
            double tw = 0.0, pw = 0.0, mw = 0.0, mf = 0.0;  // wave 0: lane i holds chunk cb + i
            if (tid < 64) {
                mw = tid < nc ? ms.cm[tid] : 0.0;
                mf = tid < nc ? ms.cmf[tid] : 0.0;
                tw = wave_find(mw, 0.0, 0.0).total;
                pw = wave_find(mf, 0.0, 0.0).total;
            }
            bool fallback = false;
            double tot = 0.0;
            if (!cluster_step(slots, R, W, w, tag, a.spin, dbl_hi(tw), dbl_lo(tw), 0u, xs)) {
                bad = gaveup = true;
            } else {
                for (int j = 0; j < W; ++j) tot += dbl_of(xs.xp[j][0], xs.xp[j][1]);
                fallback = !(tot > 0.0);
                if (fallback) {
                    if (!cluster_step(slots, R + 1, W, w, tag, a.spin, dbl_hi(pw), dbl_lo(pw), 0u,
                                      xs)) {
                        bad = gaveup = true;
                    } else {
                        tot = 0.0;
                        for (int j = 0; j < W; ++j) tot += dbl_of(xs.xp[j][0], xs.xp[j][1]);
                    }
                }
            }
            if (!bad) {
                // the owner: the first member with a positive total whose inclusive prefix
                // reaches t, else (rounding) the last positive one
                const double t = (double)uG * tot;
                int owner = -1, last = -1;
                double carry = 0.0, before = 0.0, last_before = 0.0;
                for (int j = 0; j < W; ++j) {
                    const double tj = dbl_of(xs.xp[j][0], xs.xp[j][1]);
                    if (tj > 0.0) {
                        if (owner < 0 && t <= carry + tj) {
                            owner = j;
                            before = carry;
                        }
                        last = j;
                        last_before = carry;
                    }
                    carry += tj;
                }
                if (owner < 0) {
                    owner = last;
                    before = last_before;
                }
                if (w == owner && tid < 64) {
                    const double t1 = t - before;
                    const Found f = wave_find(fallback ? mf : mw, t1, 0.0);
                    const int cl = f.hit >= 0 ? f.hit : f.last;
                    const double bc = f.hit >= 0 ? f.before : f.last_before;
                    int y = -1;
                    float ly = 0.f;
                    if (cl >= 0)
                        draw_in_chunk<T, false>(a, st, Wp, rowp, qrow, b, cb + cl, t1 - bc,
                                                fallback, y, ly);
                    if (tid == 0) {
                        a.out_tokens[st.out] = y;
                        if (a.probs)
                            a.probs[st.out] =
                                y >= 0 ? (float)(exp(((double)ly - (double)st.M) / st.T) / st.Z) : 0.f;
                    }
                }
                if (owner < 0 && w == 0 && tid == 0) {  // no positive weight anywhere
                    a.out_tokens[st.out] = -1;
                    if (a.probs) a.probs[st.out] = 0.f;
                }
            }
        }
    }
    if (w == 0) {  // workgroup 0 of the cluster writes the request's outputs
        for (int e = tid; e < R; e += kBlock) {
            if (e == k && !bad) continue;  // slot k is written by the final draw
            a.out_tokens[(size_t)b * R + e] = (!bad && e < k) ? a.tokens[(size_t)b * G + e] : -1;
            if (a.probs) a.probs[(size_t)b * R + e] = (!bad && e < k) ? sp[e] : 0.f;
        }
        if (tid == 0) store_state(a.dstate + b, st);
    }
    walk_end(hdr, epoch, b, w, W, gaveup, bad ? -1 : k, a.accept_len);
}

// k_tree_walk: the target-only token-tree walk, one cluster of W workgroups per request
// (blockIdx = b * W + w, workgroup w owning a slice of whole fine chunks of every row).
// Only the rows of the nodes the walk reaches are read.  At each node the slices' row
// statistics (sampling: max and normaliser; greedy: max and lowest index) travel through
// the cluster hand-off and every workgroup takes the same decision.  Sampling then weighs
// its slice of the last node's row (the rejected children's tokens excluded) for
// k_draw; greedy emits the argmax itself.
struct TreeWalkSmem {
    int par[SPEC_MAX_N];
    int tok[SPEC_MAX_N];
    union {
        struct {  // validation: pointer-jumping state
            int anc[SPEC_MAX_N];
            int dep[SPEC_MAX_N];
        };
        struct {  // the walk: children of the current node, tokens to exclude
            int kids[SPEC_MAX_N];
            int excl[SPEC_MAX_N];
        };
    };
    float lx[SPEC_MAX_N];    // logit of child j's token in the current row
    int path[SPEC_MAX_N];    // accepted nodes, by depth
    float pathp[SPEC_MAX_N]; // their target probabilities (sampling)
    int wcnt[kWaves];
    int chosen;
    int nexcl;
};

template <typename T>
__global__ __launch_bounds__(kBlock) void k_tree_walk(KArgs a, int sampling, int W, int per,
                                                      unsigned* hdr, unsigned long long* xslots,
                                                      int xstride) {
    __shared__ TreeWalkSmem ts;
    __shared__ RowSmem rs;
    __shared__ XSmem xs;
    __shared__ MassSmem ms;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x / W, w = blockIdx.x - b * W;
    const int N = a.R, V = a.V, D = a.D;
    const int lo = (int)min((long)V, (long)w * per), hi = (int)min((long)V, (long)lo + per);
    unsigned long long* slots = xslots ? xslots + (size_t)b * xstride : nullptr;
    if (!slots) hdr = nullptr;  // no hand-off words, no tag
    const uint32_t epoch = walk_epoch(hdr), tag = walk_tag(epoch);
    const int32_t* par_g = a.parents + (size_t)b * N;
    const int32_t* tok_g = a.tokens + (size_t)b * N;
    const T* logits = reinterpret_cast<const T*>(a.logits);
    bool bad = false, gaveup = false;
    const float Tf = sampling ? a.temperature[b] : 1.f;
    const double Td = (double)Tf;
    const float s2 = kLog2e / Tf;

    // One step's slice pass over node `node`'s row, handed to the cluster (the wait comes
    // later, so that what does not need the row statistics overlaps the hand-off).
    auto pass = [&](int step, int node) {
        const T* rowp = logits + ((size_t)b * N + node) * V;
        if (sampling) {  // cache-allocating: the last row's slice is weighed again
            const Part r = chunk_record<T, true, false, kWalkUnroll>(rowp, lo, hi, s2, rs);
            cluster_publish(slots, step, W, w, tag, __float_as_uint(r.m), dbl_hi(r.z),
                            dbl_lo(r.z), xs);
        } else {
            const Part r = chunk_record<T, false, true, kWalkUnroll>(rowp, lo, hi, 0.f, rs);
            cluster_publish(slots, step, W, w, tag, __float_as_uint(r.m), (uint32_t)r.idx, 0u, xs);
        }
    };

    // The tree's arrays are loaded first and the root's pass runs while they arrive; the
    // tree is checked while the pass's hand-off travels.  The root row is in bounds
    // whatever the tree holds, and a request found invalid never waits for its words.
    constexpr int kPer = SPEC_MAX_N / kBlock;
    int pr[kPer], tr[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int i = tid + c * kBlock;
        pr[c] = i < N ? par_g[i] : 0;
        tr[c] = i < N ? tok_g[i] : 0;
    }
    pass(0, 0);
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int i = tid + c * kBlock;
        if (i >= N) break;
        ts.par[i] = pr[c];
        ts.tok[i] = tr[c];
        if (i == 0) {
            if (pr[c] != -1) bad = true;
        } else {
            if (pr[c] < 0 || pr[c] >= i) bad = true;
            if (tr[c] < 0 || tr[c] >= V) bad = true;
        }
    }
    if (sampling) {
        if (!(isfinite(Tf) && Tf > 0.f)) bad = true;
        for (int d = tid; d <= D; d += kBlock) {
            const float u = a.coins[(size_t)b * (D + 1) + d];
            if (!(u > 0.f && u <= 1.f)) bad = true;
        }
    }
    bad = __syncthreads_or(bad);
    if (!bad) {
        tree_depths(ts.par, N, ts.anc, ts.dep);
        for (int i = tid; i < N; i += kBlock)
            if (ts.dep[i] > D) bad = true;
        bad = __syncthreads_or(bad);
    }

    int cur = 0, d = 0, nexcl = 0, last = -1;
    float M = 0.f;
    double Z = 1.0;
    for (int step = 0; !bad; ++step) {
        const T* rowp = logits + ((size_t)b * N + cur) * V;
        // while this step's words travel: the children of cur in ascending node id (ordered
        // compaction) and, for sampling, their tokens' logits
        int count = 0;
        for (int base = cur + 1; base < N; base += kBlock) {
            const int c = base + tid;
            const bool f = c < N && ts.par[c] == cur;
            const unsigned long long m = __ballot(f);
            if (lane == 0) ts.wcnt[wave] = __popcll(m);
            __syncthreads();
            int off = count, total = 0;
            for (int q = 0; q < kWaves; ++q) {
                if (q < wave) off += ts.wcnt[q];
                total += ts.wcnt[q];
            }
            if (f) ts.kids[off + __popcll(m & ((1ull << lane) - 1ull))] = c;
            __syncthreads();
            count += total;
        }
        for (int j = tid; j < count && sampling; j += kBlock)
            ts.lx[j] = Ld<T>::one(rowp + ts.tok[ts.kids[j]]);
        if (!cluster_wait(slots, step, W, tag, a.spin, xs)) {
            bad = gaveup = true;
            break;
        }
        M = -INFINITY;
        if (sampling) {
            for (int j = 0; j < W; ++j) M = fmaxf(M, __uint_as_float(xs.xp[j][0]));
            Z = cluster_norm(xs, W, M, Td);
        } else {
            for (int j = 0; j < W; ++j) {  // slices in order: the lowest index among equal maxima
                const float mj = __uint_as_float(xs.xp[j][0]);
                if (mj > M) {
                    M = mj;
                    last = (int)xs.xp[j][1];
                }
            }
        }
        if (M == -INFINITY) {  // a row the walk reaches has no finite logit
            bad = true;
            break;
        }
        if (sampling && tid < 64) {
            // wave 0: lane i evaluates the probability of child c0 + i, 64 children at a
            // time, and every lane adds them up in child order (the same bits in all lanes)
            const double u = (double)a.coins[(size_t)b * (D + 1) + d];
            const double tha = (double)a.th_acc, ths = (double)a.th_single;
            double acc = 0.0, pch = 0.0;
            int ch = -1;
            for (int c0 = 0; c0 < count && ch < 0; c0 += 64) {
                const int j = c0 + lane;
                const double mine = j < count ? (double)ex2((ts.lx[j] - M) * s2) / Z : 0.0;
                const int n = min(64, count - c0);
                for (int e = 0; e < n; ++e) {
                    const double pc = lane_dbl(mine, e);
                    acc += pc;
                    if (u <= acc / tha || pc >= ths) {
                        ch = c0 + e;
                        pch = pc;
                        break;
                    }
                }
            }
            if (tid == 0) {
                ts.chosen = ch;
                if (ch >= 0) {
                    ts.path[d] = ts.kids[ch];
                    ts.pathp[d] = (float)pch;
                }
            }
        }
        if (!sampling && tid == 0) {  // greedy: the child whose token is the argmax
            int ch = -1;
            for (int j = 0; j < count; ++j)
                if (ts.tok[ts.kids[j]] == last) {
                    ch = j;
                    break;
                }
            ts.chosen = ch;
            if (ch >= 0) ts.path[d] = ts.kids[ch];
        }
        __syncthreads();
        const int ch = ts.chosen;
        __syncthreads();
        if (ch < 0) {  // a leaf, or no child accepted: the walk stops at cur
            if (sampling && tid < 64) {  // the children tried, each token once, in child order
                // wave 0, 64 children at a time: a child is listed when no earlier child has
                // its token; the listed ones keep their order (ballot prefix)
                int n = 0;
                for (int c0 = 0; c0 < count; c0 += 64) {
                    const int j = c0 + lane;
                    const int t = j < count ? ts.tok[ts.kids[j]] : -1;
                    bool first = j < count;
                    for (int e = 0; e < j && first; ++e) first = ts.tok[ts.kids[e]] != t;
                    const unsigned long long m = __ballot(first);
                    if (first) ts.excl[n + __popcll(m & ((1ull << lane) - 1ull))] = t;
                    n += __popcll(m);
                }
                if (tid == 0) ts.nexcl = n;
            }
            __syncthreads();
            nexcl = sampling ? ts.nexcl : 0;
            break;
        }
        cur = ts.kids[ch];
        ++d;
        pass(step + 1, cur);
    }

    DrawState st = {};
    st.kind = kDrawNone;
    if (!bad && sampling) {
        st.kind = kDrawTarget;
        st.row = b * N + cur;
        st.out = b * (D + 1) + d;
        st.coin = b * (D + 1) + D;
        st.nexcl = nexcl;
        st.cq = 1.f;
        st.M = M;
        st.Z = Z;
        st.invZ = (float)(1.0 / Z);
        st.T = Td;
        const T* rowp = logits + (size_t)st.row * V;
        const void* qrow;
        const WParams Wp = draw_params<T, false>(a, st, qrow);
        mass_slice<T, false>(a, st, Wp, rowp, qrow, b, lo / kFine, (hi + kFine - 1) / kFine, ms,
                             ts.excl);
    }
    if (w != 0) {  // workgroup 0 of the cluster writes the request's outputs
        walk_end(hdr, epoch, b, w, W, gaveup, 0, a.accept_len);
        return;
    }
    int32_t* out = a.out_tokens + (size_t)b * (D + 1);
    int32_t* nodes = a.accepted_nodes + (size_t)b * D;
    float* probs = a.probs ? a.probs + (size_t)b * (D + 1) : nullptr;
    if (sampling)
        for (int e = tid; e < nexcl && !bad; e += kBlock) a.excl[(size_t)b * SPEC_MAX_N + e] = ts.excl[e];
    for (int e = tid; e <= D; e += kBlock) {
        if (bad) {
            out[e] = -1;
            if (e < D) nodes[e] = -1;
            if (probs) probs[e] = 0.f;
            continue;
        }
        if (e < d) {
            out[e] = ts.tok[ts.path[e]];
            nodes[e] = ts.path[e];
            if (probs) probs[e] = sampling ? ts.pathp[e] : 0.f;
        } else if (e == d) {
            if (!sampling) {  // greedy: the argmax of the last row (sampling: the final draw)
                out[e] = last;
                if (probs) probs[e] = 0.f;
            }
        } else {
            out[e] = -1;
            if (probs) probs[e] = 0.f;
        }
        if (e >= d && e < D) nodes[e] = -1;
    }
    if (tid == 0 && sampling) store_state(a.dstate + b, st);
    walk_end(hdr, epoch, b, w, W, gaveup, bad ? -1 : d, a.accept_len);
}

// Residual mass of a row slice, sum over [lo, hi) of max(0, p_v - cq q_v) with the draw
// kernels' weights (p_v = exp2((l_v - M) * s2) * invZ in fp32), fp32 sums of four-element
// groups added in fp64; block-wide, every lane gets the same bits.
template <typename T>
__device__ double slice_resid_sum(const T* rowp, const float* qrow, int lo, int hi, float M,
                                  float s2, float invZ, float cq, RowSmem& rs) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double acc = 0.0;
    int done = lo;
    if (((uintptr_t)(rowp + lo)) % (4 * sizeof(T)) == 0 && ((uintptr_t)(qrow + lo)) % 16 == 0) {
        const int nq = (hi - lo) / 4;
        const Quad<T>* lq = reinterpret_cast<const Quad<T>*>(rowp + lo);
        const u32x4* qq = reinterpret_cast<const u32x4*>(qrow + lo);
        typedef typename Quad<T>::Raw LR;
        // a batch: quads i0 + u * kBlock + tid, u < 4, summed in fp32, added in fp64
        auto weigh = [&](const LR* lr, const u32x4* qr, int i0) {
            float bs = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (i0 + u * kBlock + tid < nq) {
                    float l[4];
                    Quad<T>::unpack(lr[u], l);
                    const float qv[4] = {__uint_as_float(qr[u].x), __uint_as_float(qr[u].y),
                                         __uint_as_float(qr[u].z), __uint_as_float(qr[u].w)};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        bs += fmaxf(ex2((l[e] - M) * s2) * invZ - cq * qv[e], 0.f);
                }
            }
            acc += (double)bs;
        };
        auto load = [&](LR* lr, u32x4* qr, int i0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                lr[u] = lq[i0 + u * kBlock + tid].raw;
                qr[u] = ld_stream(qq + i0 + u * kBlock + tid);
            }
        };
        // Full batches (every lane in range) with the next one in flight while one is
        // weighed: two named buffers take turns, and the next batch is loaded
        // unconditionally (past the last full batch it re-reads the current one), so the
        // compiler waits only for the batch it is about to weigh.
        const int step = 4 * kBlock;
        const int nfull = nq / step * step;
        int i0 = 0;
        if (nfull > 0) {
            LR la[4], lb[4];
            u32x4 qa[4], qb[4];
            load(la, qa, 0);
            for (;;) {
                load(lb, qb, i0 + step < nfull ? i0 + step : i0);
                __builtin_amdgcn_sched_barrier(0);
                weigh(la, qa, i0);
                i0 += step;
                if (i0 >= nfull) break;
                load(la, qa, i0 + step < nfull ? i0 + step : i0);
                __builtin_amdgcn_sched_barrier(0);
                weigh(lb, qb, i0);
                i0 += step;
                if (i0 >= nfull) break;
            }
        }
        if (i0 < nq) {  // the partial last batch
            LR lr[4];
            u32x4 qr[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kBlock + tid;
                if (i < nq) {
                    lr[u] = lq[i].raw;
                    qr[u] = ld_stream(qq + i);
                }
            }
            weigh(lr, qr, i0);
        }
        done = lo + nq * 4;
    }
    for (int j = done + tid; j < hi; j += kBlock) {
        const float p = ex2((Ld<T>::one(rowp + j) - M) * s2) * invZ;
        acc += (double)fmaxf(p - cq * qrow[j], 0.f);
    }
    acc = wave_sum(acc);
    if (lane == 0) rs.rz[wave] = acc;
    __syncthreads();
    double r = rs.rz[0];
    for (int q = 1; q < kWaves; ++q) r += rs.rz[q];
    __syncthreads();  // rs is reused by the next pass
    return r;
}

// k_mss_walk: a token tree verified by multi-step speculative sampling with draft rows,
// one cluster of W workgroups per request (blockIdx = b * W + w, workgroup w owning a slice
// of whole fine chunks of every row).  Only the rows the walk reaches are read.
//
// At node cur the slices' (max, normaliser) travel through the cluster hand-off.  The
// children are tested in ascending node id.  After r rejections the node's distribution
// is p^(r) = max(0, p - c_r q) / N_r, with c_0 = 0 and N_0 = 1; on the next rejection
// c_{r+1} = c_r + N_r and N_{r+1} = sum_v max(0, p_v - c_{r+1} q_v).  This holds because
// all children share one draft row q: the repeated residual norm(max(0, p^(r) - q))
// collapses to one coefficient on q (where p - c_r q <= 0 the next residual is 0 too).  So
// each rejection costs one pass over the (target, draft) slices and one hand-off, and no
// vector is kept.  c is rounded to fp32 once per step and that value is used everywhere.
//
// Child x is accepted iff p^(r)(x) > 0 and its coin <= p^(r)(x) / q(x) (q(x) = 0: iff
// p^(r)(x) > 0).  When every child is rejected each member weighs its slice of
// max(0, p - c_R q) for k_draw; at a leaf, or when a residual has no mass left, it weighs
// plain p.
struct MssWalkSmem {
    int par[SPEC_MAX_N];
    int tok[SPEC_MAX_N];
    union {
        struct {  // validation: pointer-jumping state
            int anc[SPEC_MAX_N];
            int dep[SPEC_MAX_N];
        };
        int kids[SPEC_MAX_N];  // the walk: children of the current node
    };
    float qx[SPEC_MAX_N];     // q_parent(token of node c), by node id
    float lx[SPEC_MAX_N];     // logit of child j's token in the current row
    int path[SPEC_MAX_N];     // accepted nodes, by depth
    float pathp[SPEC_MAX_N];  // their target probabilities
    int wcnt[kWaves];
    int flag;
};

template <typename T>
__global__ __launch_bounds__(kBlock) void k_mss_walk(KArgs a, int W, int per, unsigned* hdr,
                                                     unsigned long long* xslots, int xstride) {
    __shared__ MssWalkSmem sm;
    __shared__ RowSmem rs;
    __shared__ XSmem xs;
    __shared__ MassSmem2 ms;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x / W, w = blockIdx.x - b * W;
    const int N = a.R, V = a.V, D = a.D;
    const int lo = (int)min((long)V, (long)w * per), hi = (int)min((long)V, (long)lo + per);
    unsigned long long* slots = xslots ? xslots + (size_t)b * xstride : nullptr;
    if (!slots) hdr = nullptr;  // no hand-off words, no tag
    const uint32_t epoch = walk_epoch(hdr), tag = walk_tag(epoch);
    const int32_t* par_g = a.parents + (size_t)b * N;
    const int32_t* tok_g = a.tokens + (size_t)b * N;
    const float* coins = a.coins + (size_t)b * N;
    const T* logits = reinterpret_cast<const T*>(a.logits);
    bool bad = false, gaveup = false;
    const float Tf = a.temperature[b];
    const double Td = (double)Tf;
    const float s2 = kLog2e / Tf;
    int step = 0;  // the next hand-off step

    // A node's slice pass, handed to the cluster; the wait comes later, so that what does
    // not need the row statistics overlaps the hand-off.
    auto pass = [&](int node) {
        const T* rowp = logits + ((size_t)b * N + node) * V;
        // cache-allocating: a node's residual sums and final weights read its row again
        const Part r = chunk_record<T, true, false, kWalkUnroll>(rowp, lo, hi, s2, rs);
        cluster_publish(slots, step, W, w, tag, __float_as_uint(r.m), dbl_hi(r.z), dbl_lo(r.z), xs);
    };

    // The tree's arrays are loaded first and the root's pass runs while they arrive; the
    // tree is checked, and the drafted tokens' q values gathered, while the root's
    // hand-off travels.  The root row is in bounds whatever the tree holds, and a request
    // found invalid never waits for its words.
    constexpr int kPer = SPEC_MAX_N / kBlock;
    int pr[kPer], tr[kPer];
    float ur[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int i = tid + c * kBlock;
        pr[c] = i < N ? par_g[i] : 0;
        tr[c] = i < N ? tok_g[i] : 0;
        ur[c] = i < N ? coins[i] : 1.f;
    }
    pass(0);
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int i = tid + c * kBlock;
        if (i >= N) break;
        sm.par[i] = pr[c];
        sm.tok[i] = tr[c];
        if (i == 0) {
            if (pr[c] != -1) bad = true;
        } else {
            if (pr[c] < 0 || pr[c] >= i) bad = true;
            if (tr[c] < 0 || tr[c] >= V) bad = true;
        }
        if (!(ur[c] > 0.f && ur[c] <= 1.f)) bad = true;
    }
    if (!(isfinite(Tf) && Tf > 0.f)) bad = true;
    bad = __syncthreads_or(bad);
    if (!bad) {  // depths, and q of every child's token under its parent's draft row
        tree_depths(sm.par, N, sm.anc, sm.dep);
        for (int i = tid; i < N; i += kBlock) {
            if (sm.dep[i] > D) bad = true;
            if (i > 0) {
                const float q = a.q[((size_t)b * N + sm.par[i]) * V + sm.tok[i]];
                sm.qx[i] = q;
                if (!(q >= 0.f && isfinite(q))) bad = true;
            }
        }
        bad = __syncthreads_or(bad);
    }

    int cur = 0, d = 0;
    int kind = kDrawTarget;
    float cq = 0.f, M = 0.f;
    double Z = 1.0;
    while (!bad) {
        const T* rowp = logits + ((size_t)b * N + cur) * V;
        // while cur's words travel: its children in ascending node id (ordered compaction)
        // and their tokens' logits
        int count = 0;
        for (int base = cur + 1; base < N; base += kBlock) {
            const int c = base + tid;
            const bool f = c < N && sm.par[c] == cur;
            const unsigned long long m = __ballot(f);
            if (lane == 0) sm.wcnt[wave] = __popcll(m);
            __syncthreads();
            int off = count, total = 0;
            for (int q = 0; q < kWaves; ++q) {
                if (q < wave) off += sm.wcnt[q];
                total += sm.wcnt[q];
            }
            if (f) sm.kids[off + __popcll(m & ((1ull << lane) - 1ull))] = c;
            __syncthreads();
            count += total;
        }
        for (int j = tid; j < count; j += kBlock) sm.lx[j] = Ld<T>::one(rowp + sm.tok[sm.kids[j]]);
        {
            if (!cluster_wait(slots, step++, W, tag, a.spin, xs)) {
                bad = gaveup = true;
                break;
            }
            M = -INFINITY;
            for (int k = 0; k < W; ++k) M = fmaxf(M, __uint_as_float(xs.xp[k][0]));
            Z = cluster_norm(xs, W, M, Td);
        }
        if (M == -INFINITY) {  // a row on the walk with no finite logit
            bad = true;
            break;
        }
        kind = kDrawTarget;
        cq = 0.f;
        if (count == 0) break;  // a leaf: the bonus from its own row
        const float* qrow = a.q + ((size_t)b * N + cur) * V;
        const float invZ = (float)(1.0 / Z);
        double c = 0.0, Nr = 1.0;
        int chosen = -1;
        for (int j = 0; j < count; ++j) {
            const int child = sm.kids[j];
            if (tid == 0) {
                const double px = (double)ex2((sm.lx[j] - M) * s2) / Z;
                const double qx = (double)sm.qx[child];
                double pr = px - c * qx;
                pr = pr > 0.0 ? pr / Nr : 0.0;
                const double u = (double)coins[child - 1];
                const bool acc = qx > 0.0 ? (pr > 0.0 && u <= pr / qx) : pr > 0.0;
                sm.flag = acc;
                if (acc) {
                    sm.path[d] = child;
                    sm.pathp[d] = (float)px;
                }
            }
            __syncthreads();
            const bool accepted = sm.flag != 0;
            __syncthreads();
            if (accepted) {
                chosen = child;
                break;
            }
            const double cn = (double)(float)(c + Nr);
            if (j == count - 1) {  // every child rejected: the final residual
                kind = kDrawResidual;
                cq = (float)cn;
                break;
            }
            const double Nw = slice_resid_sum<T>(rowp, qrow, lo, hi, M, s2, invZ, (float)cn, rs);
            if (!cluster_step(slots, step++, W, w, tag, a.spin, dbl_hi(Nw), dbl_lo(Nw), 0u, xs)) {
                bad = gaveup = true;
                break;
            }
            double Nn = 0.0;
            for (int k = 0; k < W; ++k) Nn += dbl_of(xs.xp[k][0], xs.xp[k][1]);
            if (!(Nn > 0.0)) break;  // no residual mass left: draw from the target row
            c = cn;
            Nr = Nn;
        }
        if (bad || chosen < 0) break;
        cur = chosen;
        ++d;
        pass(cur);
    }

    DrawState st = {};
    st.kind = kDrawNone;
    if (!bad) {
        st.kind = kind;
        st.row = b * N + cur;
        st.qrow = b * N + cur;
        st.out = b * (D + 1) + d;
        st.coin = b * N + N - 1;
        st.nexcl = 0;
        st.cq = cq;
        st.M = M;
        st.Z = Z;
        st.invZ = (float)(1.0 / Z);
        st.T = Td;
        const T* rowp = logits + (size_t)st.row * V;
        const void* qrow;
        const WParams Wp = draw_params<T, false>(a, st, qrow);
        mass_slice2<T, false>(a, st, Wp, rowp, qrow, b, lo / kFine, (hi + kFine - 1) / kFine, ms,
                             nullptr);
    }
    if (w != 0) {  // workgroup 0 of the cluster writes the request's outputs
        walk_end(hdr, epoch, b, w, W, gaveup, 0, a.accept_len);
        return;
    }
    int32_t* out = a.out_tokens + (size_t)b * (D + 1);
    int32_t* nodes = a.accepted_nodes + (size_t)b * D;
    float* probs = a.probs ? a.probs + (size_t)b * (D + 1) : nullptr;
    for (int e = tid; e <= D; e += kBlock) {
        if (bad) {
            out[e] = -1;
            if (e < D) nodes[e] = -1;
            if (probs) probs[e] = 0.f;
            continue;
        }
        if (e < d) {  // slot d is written by the final draw
            out[e] = sm.tok[sm.path[e]];
            nodes[e] = sm.path[e];
            if (probs) probs[e] = sm.pathp[e];
        } else if (e > d) {
            out[e] = -1;
            if (probs) probs[e] = 0.f;
        }
        if (e >= d && e < D) nodes[e] = -1;
    }
    if (tid == 0) store_state(a.dstate + b, st);
    walk_end(hdr, epoch, b, w, W, gaveup, bad ? -1 : d, a.accept_len);
}

// One wave per request: chunk, then segment, then token.
template <typename T, bool kFilt>
__global__ __launch_bounds__(64) void k_draw(KArgs a) {
    const int lane = threadIdx.x;
    const int S2 = a.S2, V = a.V;
    const int b = blockIdx.x;
    // the first 64 chunk masses and the request's last coin (the final draw's) do not depend
    // on the draw state: read them alongside it
    const double m0 = lane < S2 ? a.mass[(size_t)b * S2 + lane] : 0.0;
    const bool coin_known = a.coins != nullptr && a.coin_stride > 0;
    const float u0 = coin_known ? a.coins[(size_t)b * a.coin_stride + a.coin_stride - 1] : 0.f;
    const DrawState st = load_state(a.dstate + b);
    if (st.kind == kDrawNone) return;
    const T* rowp = reinterpret_cast<const T*>(a.logits) + (size_t)st.row * V;
    const void* qrow;
    const WParams W = draw_params<T, kFilt>(a, st, qrow);
    const double u = (double)(coin_known ? u0 : a.coins[st.coin]);
    double tot = wave_sum(m0);
    for (int i0 = 64; i0 < S2; i0 += 64)
        tot += wave_sum(i0 + lane < S2 ? a.mass[(size_t)b * S2 + i0 + lane] : 0.0);
    const bool fallback = !(tot > 0.0);  // plain target weights, nothing excluded
    if (fallback) {
        tot = 0.0;
        for (int i0 = 0; i0 < S2; i0 += 64)
            tot += wave_sum(i0 + lane < S2 ? a.massfb[(size_t)b * S2 + i0 + lane] : 0.0);
    }
    int y = -1;
    float ly = 0.f;
    const double t = u * tot;
    double before = 0.0;
    int c;
    if (!fallback && S2 <= 64) {  // the masses are in registers already (as wave_locate finds)
        const Found f = wave_find(m0, t, 0.0);
        c = f.hit >= 0 ? f.hit : f.last;
        before = f.hit >= 0 ? f.before : f.last_before;
    } else {
        c = wave_locate((fallback ? a.massfb : a.mass) + (size_t)b * S2, S2, t, before);
    }
    if (c >= 0) draw_in_chunk<T, kFilt>(a, st, W, rowp, qrow, b, c, t - before, fallback, y, ly);
    if (lane == 0) {
        a.out_tokens[st.out] = y;
        if (a.probs)
            a.probs[st.out] = y >= 0 ? (float)(exp(((double)ly - (double)st.M) / st.T) / st.Z) : 0.f;
    }
}

// ---------------------------------------------------------------------------------------
// k_filter_rows: one workgroup per logit row of a filtered chain call (every target row,
// then every draft row) -- the row max and normaliser at the request's temperature, then
// the top-k and top-p thresholds by radix selection over order-preserving keys
//
// Each selection walks the key from its top digit down: a histogram pass counts and
// weighs (fixed point, so sums are exact and independent of order) the tokens that
// agree with the digits chosen so far, and the walk takes the digit where the count
// (top-k) or mass (top-p) accumulated from the largest keys reaches what is needed.
// bf16 keys have 16 significant bits (two 8-bit digits); fp32 keys take four.

constexpr int kHistBins = 256;  // 8-bit radix digits

constexpr int kCandCap = 2048;  // top-k candidates kept in LDS by the direct selection
constexpr int kItemCap = 1024;  // recorded batches the candidate pass can list

struct FilterSmem {
    RowSmem rs;
    union {
        struct {
            uint32_t cnt[kWaves][kHistBins];  // one private histogram per wave
            unsigned long long mass[kWaves][kHistBins];
        };
        alignas(16) uint32_t cand[kCandCap];  // direct selection: candidate keys
    };
    alignas(16) uint32_t lanekey[kBlock];  // lane maxima's keys; then the sorted candidates (n <= kBlock)
    uint16_t bkey[kMaxBatchRec * kBlock];  // batch maxima of the first pass (key top bits)
    uint16_t item[kItemCap];               // the batches the candidate pass reads (j * kBlock + t)
    uint32_t candidx[kBlock];              // the first kBlock candidates' token ids
    int ncand;
    int nkept;
    unsigned long long wtot[3][kWaves];
    int pick_thread;
    int last_thread;
    int pick;
    uint32_t lbkey;  // direct selection: the k-th largest lane maximum's key
    unsigned long long above_cnt, above_mass, bucket_mass, total_cnt, total_mass;
    double need_mass;
};

template <typename T>
struct Digits;
template <>
struct Digits<uint16_t> {  // a widened bf16 has 16 significant key bits
    static constexpr int kLevels = 2;
    __device__ static int shift(int l) { return 24 - 8 * l; }
};
template <>
struct Digits<float> {
    static constexpr int kLevels = 4;
    __device__ static int shift(int l) { return 24 - 8 * l; }
};

// Exclusive block scan of three u64 values at once (every thread gets its offsets and
// the totals).
__device__ inline void block_scan3(unsigned long long v[3], unsigned long long ex[3],
                                   unsigned long long tot[3], FilterSmem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned long long inc[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        unsigned long long x = v[k];
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        inc[k] = x;
        if (lane == 63) sm.wtot[k][wave] = x;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        unsigned long long off = 0, all = 0;
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) off += sm.wtot[k][w];
            all += sm.wtot[k][w];
        }
        ex[k] = off + inc[k] - v[k];
        tot[k] = all;
    }
    __syncthreads();
}

// One histogram pass: the tokens with key >= lo whose key agrees with `prefix` on the
// bits of `pmask` are counted and weighed (fixed point) by digit (key >> shift) & 255,
// each wave into its own LDS histogram; the four are added up at the end.
template <typename T>
__device__ void hist_pass(const T* rowp, int V, float M, float s2, float fscale, uint32_t lo,
                          uint32_t prefix, uint32_t pmask, int shift, FilterSmem& sm) {
    const int tid = threadIdx.x, wave = tid >> 6;
    constexpr int kVec = Ld<T>::kVec;
    for (int i = tid; i < kWaves * kHistBins; i += kBlock) {
        (&sm.cnt[0][0])[i] = 0u;
        (&sm.mass[0][0])[i] = 0ull;
    }
    __syncthreads();
    uint32_t* cnt = sm.cnt[wave];
    unsigned long long* mass = sm.mass[wave];
    auto visit = [&](float x) {
        const uint32_t key = order_key(x);
        if (key >= lo && (key & pmask) == prefix) {
            const uint32_t dg = (key >> shift) & (uint32_t)(kHistBins - 1);
            atomicAdd(&cnt[dg], 1u);
            atomicAdd(&mass[dg], (unsigned long long)(ex2((x - M) * s2) * fscale));
        }
    };
    int head = (int)(((16u - ((uint32_t)(uintptr_t)rowp & 15u)) & 15u) / sizeof(T));
    if (head > V) head = V;
    const int nv = (V - head) / kVec;
    const int tail0 = head + nv * kVec;
    if (tid < head) visit(Ld<T>::one(rowp + tid));
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + head);
    int v = tid;
    for (; v + kBlock < nv; v += 2 * kBlock) {
        const u32x4 r0 = ld_stream(vp + v), r1 = ld_stream(vp + v + kBlock);
        float f[2 * kVec];
        Ld<T>::unpack(r0, f);
        Ld<T>::unpack(r1, f + kVec);
#pragma unroll
        for (int e = 0; e < 2 * kVec; ++e) visit(f[e]);
    }
    for (; v < nv; v += kBlock) {
        float f[kVec];
        Ld<T>::unpack(ld_stream(vp + v), f);
#pragma unroll
        for (int e = 0; e < kVec; ++e) visit(f[e]);
    }
    if (tail0 + tid < V) visit(Ld<T>::one(rowp + tail0 + tid));
    __syncthreads();
    for (int d = tid; d < kHistBins; d += kBlock) {
        for (int w = 1; w < kWaves; ++w) {
            sm.cnt[0][d] += sm.cnt[w][d];
            sm.mass[0][d] += sm.mass[w][d];
        }
    }
    __syncthreads();
}

// The digit, scanning from the top, at which the accumulated count (by_mass false) or
// mass reaches `need` (the lowest non-empty digit if it never does).  Updates the
// count / mass above the chosen digit and leaves the chosen digit's mass in
// sm.bucket_mass; the level's totals go to sm.total_cnt / sm.total_mass.
__device__ int hist_pick(int nb, bool first, bool by_mass, double need_frac,
                         unsigned long long need_cnt, FilterSmem& sm) {
    const int tid = threadIdx.x;
    const int per = nb >= kBlock ? nb / kBlock : 1;
    const int hi = nb - 1 - tid * per;  // this thread owns digits hi, hi-1, .., hi-per+1
    const bool owns = tid * per < nb;
    unsigned long long v[3] = {0ull, 0ull, 0ull}, ex[3], tot[3];
    if (owns)
        for (int d = hi; d > hi - per; --d) {
            v[0] += sm.cnt[0][d];
            v[1] += sm.mass[0][d];
        }
    v[2] = by_mass ? v[1] : v[0];
    block_scan3(v, ex, tot, sm);
    const unsigned long long base_sel = by_mass ? sm.above_mass : sm.above_cnt;
    // by mass the need is a fraction of every candidate's mass, which only the first level
    // sees (it is fixed there and kept); by count it is given
    if (first && tid == 0) sm.need_mass = need_frac * (double)tot[1];
    __syncthreads();
    const double need = by_mass ? sm.need_mass : (double)need_cnt;
    if (tid == 0) {
        sm.pick_thread = INT_MAX;
        sm.last_thread = -1;
        sm.pick = 0;
        sm.bucket_mass = 0ull;
    }
    __syncthreads();
    if (owns && v[0] > 0) {
        if ((double)(base_sel + ex[2] + v[2]) >= need) atomicMin(&sm.pick_thread, tid);
        atomicMax(&sm.last_thread, tid);
    }
    __syncthreads();
    const int who = sm.pick_thread != INT_MAX ? sm.pick_thread : sm.last_thread;
    if (tid == who) {
        unsigned long long ac = sm.above_cnt + ex[0], am = sm.above_mass + ex[1];
        int pick = -1;
        for (int d = hi; d > hi - per; --d) {
            if (sm.cnt[0][d] == 0u) continue;
            const unsigned long long sel = by_mass ? am + sm.mass[0][d] : ac + sm.cnt[0][d];
            pick = d;
            if (sm.pick_thread != INT_MAX && (double)sel >= need) break;
            ac += sm.cnt[0][d];
            am += sm.mass[0][d];
        }
        if (sm.pick_thread == INT_MAX) {  // never reached: keep every candidate
            ac -= sm.cnt[0][pick];
            am -= sm.mass[0][pick];
        }
        sm.pick = pick;
        sm.above_cnt = ac;
        sm.above_mass = am;
        sm.bucket_mass = sm.mass[0][pick];
    }
    if (tid == 0) {
        sm.total_cnt = tot[0];
        sm.total_mass = tot[1];
    }
    __syncthreads();
    return sm.pick;
}

// Radix selection of a threshold key t over the row's tokens with key >= lo: the largest
// t whose keys >= t number at least need_cnt (top-k) or weigh at least need_frac of the
// candidates' mass (top-p).  Returns t; *kept = fixed-point mass of the keys >= t.
template <typename T>
__device__ uint32_t radix_select(const T* rowp, int V, float M, float s2, float fscale,
                                 uint32_t lo, bool by_mass, double need_frac,
                                 unsigned long long need_cnt, unsigned long long* kept,
                                 FilterSmem& sm) {
    if (threadIdx.x == 0) {
        sm.above_cnt = 0ull;
        sm.above_mass = 0ull;
    }
    __syncthreads();
    uint32_t prefix = 0u, pmask = 0u;
    for (int l = 0; l < Digits<T>::kLevels; ++l) {
        const int shift = Digits<T>::shift(l);
        hist_pass<T>(rowp, V, M, s2, fscale, lo, prefix, pmask, shift, sm);
        const int d = hist_pick(kHistBins, l == 0, by_mass, need_frac, need_cnt, sm);
        prefix |= (uint32_t)d << shift;
        pmask |= (uint32_t)(kHistBins - 1) << shift;
    }
    *kept = sm.above_mass + sm.bucket_mass;
    return prefix;
}

// Block-wide bitonic sort of a[0..n) (n a power of two) into descending order.
__device__ void bitonic_desc(uint32_t* a, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            __syncthreads();
            for (int t = threadIdx.x; t < n / 2; t += kBlock) {
                const int lo = 2 * t - (t & (stride - 1));  // the pair (lo, lo + stride)
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint32_t x = a[lo], y = a[hi];
                if (desc ? x < y : x > y) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
        }
    }
    __syncthreads();
}

__device__ inline float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Descending rank of this thread's key among the n keys a[0..n) (this thread's being a[i]):
// the keys above it, plus the equal keys at lower positions, so the ranks of the n keys
// are 0..n-1 without repeats, and placing each key at its rank sorts them descending.
// `a` is 16-byte aligned; the keys are read four at a time.
__device__ inline int desc_rank(const uint32_t* a, int n, int i, uint32_t key) {
    auto above = [&](uint32_t o, int j) { return (o > key) | ((o == key) & (j < i)); };
    int r = 0;
    const int n4 = n & ~3;
#pragma unroll 8
    for (int j = 0; j < n4; j += 4) {
        const uint4 o = *reinterpret_cast<const uint4*>(a + j);
        r += above(o.x, j) + above(o.y, j + 1) + above(o.z, j + 2) + above(o.w, j + 3);
    }
    for (int j = n4; j < n; ++j) r += above(a[j], j);
    return r;
}

// The wave's 64 keys sorted in descending order across its lanes (lane 0 the largest), by
// a bitonic network of cross-lane exchanges.
__device__ inline uint32_t wave_sort_desc(uint32_t key) {
    const int lane = threadIdx.x & 63;
    for (int size = 2; size <= 64; size <<= 1) {
        const bool desc = (lane & size) == 0;  // this lane's block of `size` runs descending
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint32_t other = (uint32_t)__shfl_xor((int)key, stride);
            const bool lower = (lane & stride) == 0;
            key = (lower == desc) ? max(key, other) : min(key, other);
        }
    }
    return key;
}

// Number of entries of the descending list a[0..64) above `key` (strict: > key; else >= key).
__device__ inline int count_above(const uint32_t* a, uint32_t key, bool strict) {
    int lo = 0, hi = 64;  // a[i] is above key for every i < lo, for no i >= hi
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const bool above = strict ? a[mid] > key : a[mid] >= key;
        if (above)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// Direct top-k (k <= kBlock) then top-p on the top-k set, for rows whose candidates fit in
// LDS.  The k-th largest of the lanes' maxima (one per lane from the first pass) is a
// lower bound of the row's k-th largest logit, so one more pass collects every token at
// or above it; sorting those keys gives the k-th largest key exactly, and prefix sums of
// the fixed-point masses over the sorted keys give the top-p threshold.  Thresholds and
// kept mass are the ones the radix selection finds.  Returns false (nothing decided)
// when the candidates do not fit.
//
// The k-th lane maximum comes from ranks: each wave sorts its 64 lane maxima across its
// lanes, and a key's rank among all 256 is its place in its own wave's list plus, from
// each other wave's list, a binary search for the keys above it.  The order of at most
// kBlock candidates also comes from ranks (each thread counts the candidates above its
// own).  Either replaces a sorting network's dozens of barrier-separated stages.
//
// With `rec` the first pass left every batch's maximum in sm.bkey (a row without NaN whose
// full batches fit the record): only batches whose maximum reaches the bound are read
// again, so the row is read about once instead of twice.  Those batches are listed in LDS
// first and their loads dealt out over the whole workgroup, all in flight at once: a
// lane walking its own batches would wait one memory round trip per batch that any lane
// of its wave needs.
template <typename T>
__device__ bool direct_select(const T* rowp, int V, float M, float s2, float fscale, int k,
                              bool fp, double tp, float lane_max, bool rec, uint32_t* th_out,
                              unsigned long long* kept_out, int32_t* ids_out, FilterSmem& sm) {
    const int tid = threadIdx.x;
    constexpr int kVec = Ld<T>::kVec;
    {
        // keys ordered by value, then wave, then place in the wave: every rank is unique
        const int lane = tid & 63, wave = tid >> 6;
        const uint32_t mykey = wave_sort_desc(order_key(lane_max));
        sm.lanekey[tid] = mykey;
        if (tid == 0) sm.ncand = 0;
        __syncthreads();
        int rk = lane;
        for (int o = 0; o < kWaves; ++o)
            if (o != wave) rk += count_above(sm.lanekey + 64 * o, mykey, o > wave);
        if (rk == k - 1) sm.lbkey = mykey;  // one thread
        __syncthreads();
    }
    const uint32_t lb = sm.lbkey;
    auto visit = [&](float x, int idx) {
        const uint32_t key = order_key(x);
        if (key >= lb) {
            const int slot = atomicAdd(&sm.ncand, 1);
            if (slot < kCandCap) sm.cand[slot] = key;
            if (slot < kBlock) sm.candidx[slot] = (uint32_t)idx;
        }
    };
    int head = (int)(((16u - ((uint32_t)(uintptr_t)rowp & 15u)) & 15u) / sizeof(T));
    if (head > V) head = V;
    const int nv = (V - head) / kVec;
    const int tail0 = head + nv * kVec;
    if (tid < head) visit(Ld<T>::one(rowp + tid), tid);
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + head);
    int v = tid;
    const uint32_t lb16 = lb >> 16;  // key >= lb implies key >> 16 >= lb16
    bool listed = false;
    if (rec) {
        // this lane's full batches whose recorded maximum reaches the bound
        int nfull = 0, q = 0;
        for (int j = 0; v + (kUnroll - 1) * kBlock < nv; v += kUnroll * kBlock, ++j, ++nfull)
            if (sm.bkey[j * kBlock + tid] >= lb16) ++q;
        unsigned long long c3[3] = {(unsigned long long)q, 0ull, 0ull}, e3[3], t3[3];
        block_scan3(c3, e3, t3, sm);
        const int total = (int)t3[0];
        if (total <= kItemCap) {  // uniform: every thread has the same total
            listed = true;
            int o = (int)e3[0];
            for (int j = 0; j < nfull; ++j)
                if (sm.bkey[j * kBlock + tid] >= lb16) sm.item[o++] = (uint16_t)(j * kBlock + tid);
            __syncthreads();
            // one vector per (batch, u): up to four per thread in flight at once
            const int nvis = total * kUnroll;
            for (int base = 0; base < nvis; base += 4 * kBlock) {
                u32x4 r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int it = base + e * kBlock + tid;
                    if (it < nvis) {
                        const int bt = sm.item[it / kUnroll];
                        const int vv = (bt % kBlock) + kBlock * (kUnroll * (bt / kBlock) + it % kUnroll);
                        r[e] = ld_stream(vp + vv);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int it = base + e * kBlock + tid;
                    if (it < nvis) {
                        const int bt = sm.item[it / kUnroll];
                        const int vv = (bt % kBlock) + kBlock * (kUnroll * (bt / kBlock) + it % kUnroll);
                        float f[kVec];
                        Ld<T>::unpack(r[e], f);
#pragma unroll
                        for (int x = 0; x < kVec; ++x) visit(f[x], head + vv * kVec + x);
                    }
                }
            }
        } else {
            v = tid;  // too many to list: the batches one by one below
        }
    }
    if (!listed) {
        for (int j = 0; v + (kUnroll - 1) * kBlock < nv; v += kUnroll * kBlock, ++j) {
            if (rec && sm.bkey[j * kBlock + tid] < lb16) continue;  // nothing here reaches lb
            u32x4 r[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) r[u] = ld_stream(vp + v + u * kBlock);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float f[kVec];
                Ld<T>::unpack(r[u], f);
#pragma unroll
                for (int e = 0; e < kVec; ++e) visit(f[e], head + (v + u * kBlock) * kVec + e);
            }
        }
    }
    {
        // the fewer than kUnroll vectors after a lane's last full batch, all loads in flight
        // before the first is visited
        u32x4 r[kUnroll - 1];
#pragma unroll
        for (int u = 0; u < kUnroll - 1; ++u)
            if (v + u * kBlock < nv) r[u] = ld_stream(vp + v + u * kBlock);
#pragma unroll
        for (int u = 0; u < kUnroll - 1; ++u) {
            if (v + u * kBlock < nv) {
                float f[kVec];
                Ld<T>::unpack(r[u], f);
#pragma unroll
                for (int e = 0; e < kVec; ++e) visit(f[e], head + (v + u * kBlock) * kVec + e);
            }
        }
    }
    if (tail0 + tid < V) visit(Ld<T>::one(rowp + tail0 + tid), tail0 + tid);
    __syncthreads();
    const int n = sm.ncand;
    if (n > kCandCap) return false;  // uniform: every thread read the same count
    const uint32_t* srt;  // the candidates' keys in descending order
    if (n <= kBlock) {
        const uint32_t key = tid < n ? sm.cand[tid] : 0u;
        const int rk = tid < n ? desc_rank(sm.cand, n, tid, key) : 0;
        if (tid < n) sm.lanekey[rk] = key;  // the lane maxima are no longer needed
        __syncthreads();
        srt = sm.lanekey;
    } else {
        int n2 = 1;
        while (n2 < n) n2 <<= 1;
        for (int j = n + tid; j < n2; j += kBlock) sm.cand[j] = 0u;  // below every real key
        bitonic_desc(sm.cand, n2);
        srt = sm.cand;
    }
    const uint32_t thk = srt[k - 1];
    int nk = k;  // ties at the k-th key are kept
    while (nk < n && srt[nk] == thk) ++nk;
    // fixed-point masses over the sorted keys: lane t owns a contiguous run of them
    const int per = (nk + kBlock - 1) / kBlock;
    const int j0 = min(nk, tid * per), j1 = min(nk, j0 + per);
    unsigned long long v3[3] = {0ull, 0ull, 0ull}, ex[3], tot[3];
    for (int j = j0; j < j1; ++j)
        v3[0] += (unsigned long long)(ex2((key_value(srt[j]) - M) * s2) * fscale);
    block_scan3(v3, ex, tot, sm);
    uint32_t th = thk;
    unsigned long long kept = tot[0];
    if (fp) {
        const double need = tp * (double)tot[0];
        if (tid == 0) sm.pick = nk - 1;
        __syncthreads();
        // the first sorted position whose inclusive prefix reaches the need
        unsigned long long acc = ex[0];
        for (int j = j0; j < j1; ++j) {
            acc += (unsigned long long)(ex2((key_value(srt[j]) - M) * s2) * fscale);
            if ((double)acc >= need) {
                atomicMin(&sm.pick, j);
                break;
            }
        }
        __syncthreads();
        const int jp = sm.pick;
        th = srt[jp];
        // kept mass: every token with key >= th (ties of the threshold included)
        unsigned long long part = 0ull;
        for (int j = j0; j < j1; ++j)
            if (srt[j] >= th)
                part += (unsigned long long)(ex2((key_value(srt[j]) - M) * s2) * fscale);
        unsigned long long p3[3] = {part, 0ull, 0ull}, e3[3], t3[3];
        block_scan3(p3, e3, t3, sm);
        kept = t3[0];
    }
    *th_out = th;
    *kept_out = kept;
    if (ids_out) {
        // The kept tokens (key >= th) are all among the candidates (th >= lb).  When their
        // ids were all recorded (n <= kBlock, the candidates still in visiting order), the
        // list goes to the row's kept words; otherwise the count -1 says there is none.
        if (n <= kBlock) {
            if (tid == 0) sm.nkept = 0;
            __syncthreads();
            if (tid < n && sm.cand[tid] >= th)
                ids_out[1 + atomicAdd(&sm.nkept, 1)] = (int32_t)sm.candidx[tid];
            __syncthreads();
            if (tid == 0) ids_out[0] = sm.nkept;
        } else if (tid == 0) {
            ids_out[0] = -1;
        }
    }
    return true;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_filter_rows(KArgs a) {
    __shared__ FilterSmem sm;
    const int R = a.R, G = R - 1, V = a.V;
    const int r = blockIdx.x;
    const bool draft = r >= a.B * R;
    const int b = draft ? (r - a.B * R) / G : r / R;
    const T* rowp = draft ? reinterpret_cast<const T*>(a.dlogits) + (size_t)(r - a.B * R) * V
                          : reinterpret_cast<const T*>(a.logits) + (size_t)r * V;
    // the request's knobs are read before the pass and waited for after it
    const float Tf = a.temperature[b];
    const int k = a.top_k ? a.top_k[b] : 0;
    const float tp = a.top_p ? a.top_p[b] : 1.f;
    const float s2 = kLog2e / Tf;
    float lane_max;
    // the batch record covers every full batch of a lane when the row has at most
    // kMaxBatchRec of them (the vector count bounds it: the head shifts it by less than one)
    const long nvec = (long)V * sizeof(T) / 16;
    const bool fits = nvec / (kUnroll * kBlock) + 1 <= kMaxBatchRec;
    const Part st = chunk_record<T, true, true, kUnroll>(rowp, 0, V, s2, sm.rs, &lane_max,
                                                              fits ? sm.bkey : nullptr);
    // a target row's kept-token list (the final draw reads it instead of the row)
    int32_t* ids = !draft && a.kept ? a.kept + (size_t)r * (kBlock + 1) : nullptr;
    bool listed = false;
    FiltRow fr;
    fr.M = st.m;
    fr.th = 0u;
    fr.Z = st.z;
    const bool fk = k > 0 && k < V;
    const bool fp = tp > 0.f && tp < 1.f;
    const bool t_ok = isfinite(Tf) && Tf > 0.f;
    if (st.m != -INFINITY && t_ok && (fk || fp)) {
        const float fscale = exp2f((float)a.fixbits);
        unsigned long long kept = 0ull;
        uint32_t lo = 0u;
        const bool direct = fk && k <= kBlock &&
                            direct_select<T>(rowp, V, st.m, s2, fscale, k, fp, (double)tp,
                                             lane_max, fits && isfinite(st.z), &lo, &kept, ids, sm);
        listed = direct;
        if (!direct) {
            if (fk) lo = radix_select<T>(rowp, V, st.m, s2, fscale, 0u, false, 0.0,
                                         (unsigned long long)k, &kept, sm);
            if (fp) lo = radix_select<T>(rowp, V, st.m, s2, fscale, lo, true, (double)tp,
                                         0ull, &kept, sm);
        }
        fr.th = lo;
        fr.Z = ldexp((double)kept, -a.fixbits);
    }
    if (threadIdx.x == 0) {
        a.frows[r] = fr;
        if (ids && !listed) ids[0] = -1;
    }
}

// One workgroup per filtered chain request: the acceptance scan on the filtered rows,
// its outputs and the draw state.  When k_filter_rows listed the tokens the filter keeps in
// the drawn row, the final draw happens here from that list (every other token weighs 0,
// the draft-row residual included, as its weights are at most the target's): each listed
// token is weighed with the same fp32 weights as the full draw, the weights are put in
// ascending token order, and the token whose cumulative weight reaches u * total is found
// as k_draw finds it (the plain kept weights if the residual has no mass).  The request's
// draw state is then left empty, so k_mass and k_draw pass over it.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_filter_accept(KArgs a) {
    __shared__ Smem sm;
    __shared__ float dq[kMaxRows];
    __shared__ FiltRow fq[kMaxRows];
    __shared__ FiltRow fpp[kMaxRows];
    __shared__ int kid[kBlock];      // listed token ids, then in ascending order
    __shared__ double kw[kBlock];    // their draw weights, in that order
    __shared__ double kp[kBlock];    // their plain (filtered) target weights
    const int tid = threadIdx.x;
    const int R = a.R, G = R - 1, V = a.V;
    const int b = blockIdx.x;
    const T* logits = reinterpret_cast<const T*>(a.logits);
    const T* dlogits = reinterpret_cast<const T*>(a.dlogits);
    if (tid < R) {
        sm.u[tid] = a.coins[(size_t)b * R + tid];
        fpp[tid] = a.frows[(size_t)b * R + tid];
    }
    if (tid < G) {
        fq[tid] = a.frows[(size_t)a.B * R + (size_t)b * G + tid];
        const int xi = a.tokens[(size_t)b * G + tid];
        sm.x[tid] = xi;
        if (xi >= 0 && xi < V) {
            sm.l[tid] = Ld<T>::one(logits + ((size_t)b * R + tid) * V + xi);
            dq[tid] = Ld<T>::one(dlogits + ((size_t)b * G + tid) * V + xi);
        }
    }
    const float Tf = a.temperature[b];
    const float tp = a.top_p ? a.top_p[b] : 1.f;
    const bool t_ok = isfinite(Tf) && Tf > 0.f && tp > 0.f && !isnan(tp);
    const double Td = (double)Tf;
    __syncthreads();
    if (tid < R) {  // lane i: is everything position i consults usable, and is x_i kept?
        bool ok = fpp[tid].M != -INFINITY && sm.u[tid] > 0.f && sm.u[tid] <= 1.f;
        bool keep = false;
        if (tid < G) {
            const int xi = sm.x[tid];
            ok = ok && xi >= 0 && xi < V && fq[tid].M != -INFINITY;
            if (ok && t_ok) {
                const float l = sm.l[tid], d = dq[tid];
                const double p = order_key(l) >= fpp[tid].th
                                     ? exp(((double)l - (double)fpp[tid].M) / Td) / fpp[tid].Z
                                     : 0.0;
                const double qx = order_key(d) >= fq[tid].th
                                      ? exp(((double)d - (double)fq[tid].M) / Td) / fq[tid].Z
                                      : 0.0;
                keep = qx > 0.0 ? (p > 0.0 && (double)sm.u[tid] <= p / qx) : p > 0.0;
                sm.p[tid] = p;
            }
        }
        sm.arg[tid] = (ok ? 1 : 0) | (keep ? 2 : 0);
    }
    __syncthreads();
    if (tid == 0) {
        bool valid = t_ok;
        for (int i = 0; i < R; ++i)
            if (!(sm.arg[i] & 1)) valid = false;
        int k = G;
        for (int i = 0; i < G && valid; ++i)
            if (!(sm.arg[i] & 2)) {
                k = i;
                break;
            }
        sm.k = valid ? k : -1;
        a.accept_len[b] = sm.k;
        DrawState st = {};
        st.kind = kDrawNone;
        if (valid) {
            st.kind = k < G ? kDrawResidual : kDrawTarget;
            st.row = b * R + k;
            st.qrow = b * G + k;
            st.out = b * R + k;
            st.coin = b * R + G;
            st.nexcl = 0;
            st.cq = 1.f;
            st.M = fpp[k].M;
            st.Z = fpp[k].Z;
            st.invZ = (float)(1.0 / fpp[k].Z);
            st.T = Td;
            st.thp = fpp[k].th;
            if (k < G) {
                st.thq = fq[k].th;
                st.Mq = fq[k].M;
                st.invZq = (float)(1.0 / fq[k].Z);
            }
        }
        store_state(&sm.st, st);
    }
    __syncthreads();
    const int k = sm.k;
    {
        const DrawState st = load_state(&sm.st);
        const int kn = st.kind != kDrawNone && a.kept ? a.kept[(size_t)st.row * (kBlock + 1)] : -1;
        if (kn >= 1 && kn <= kBlock) {  // uniform: every thread read the same word
            const int32_t* ids = a.kept + (size_t)st.row * (kBlock + 1) + 1;
            const T* rowp = logits + (size_t)st.row * V;
            const void* qrow;
            const WParams Wp = draw_params<T, true>(a, st, qrow);
            const int my = tid < kn ? ids[tid] : 0x7fffffff;
            float p = 0.f, w = 0.f;
            if (tid < kn)
                w = qrow ? draw_weight<T, 2, true>(rowp, qrow, my, Wp, p)
                         : draw_weight<T, 0, true>(rowp, nullptr, my, Wp, p);
            kid[tid] = my;
            __syncthreads();
            int rk = 0;  // ascending position of this token (the ids are distinct)
            for (int j = 0; j < kn; ++j) rk += kid[j] < my ? 1 : 0;
            __syncthreads();
            if (tid < kn) {
                kid[rk] = my;
                kw[rk] = (double)w;
                kp[rk] = (double)p;
            }
            __syncthreads();
            if (tid < 64) {
                double tw = 0.0, tpl = 0.0;  // totals, added as the search adds them
                for (int i0 = 0; i0 < kn; i0 += 64) {
                    tw += wave_find(i0 + tid < kn ? kw[i0 + tid] : 0.0, 0.0, 0.0).total;
                    tpl += wave_find(i0 + tid < kn ? kp[i0 + tid] : 0.0, 0.0, 0.0).total;
                }
                const bool fallback = !(tw > 0.0);
                const double t = (double)sm.u[G] * (fallback ? tpl : tw);
                double before;
                const int e = wave_locate(fallback ? kp : kw, kn, t, before);
                if (tid == 0) {
                    const int y = e >= 0 ? kid[e] : -1;
                    a.out_tokens[st.out] = y;
                    if (a.probs) {
                        const float ly = y >= 0 ? Ld<T>::one(rowp + y) : 0.f;
                        a.probs[st.out] =
                            y >= 0 ? (float)(exp(((double)ly - (double)st.M) / st.T) / st.Z) : 0.f;
                    }
                }
            }
            if (tid == 0) {
                DrawState done = st;
                done.kind = kDrawNone;
                store_state(a.dstate + b, done);
            }
        } else if (tid == 0) {
            store_state(a.dstate + b, st);
        }
    }
    for (int i = tid; i < R; i += kBlock) {
        int t = -1;
        float pr = 0.f;
        if (k >= 0 && i < k) {
            t = sm.x[i];
            pr = (float)sm.p[i];
        }
        if (i != k) {  // slot k is written by the final draw
            a.out_tokens[(size_t)b * R + i] = t;
            if (a.probs) a.probs[(size_t)b * R + i] = pr;
        }
    }
}

// ---------------------------------------------------------------------------------------
// k_tree_mask: one workgroup per request -- the ancestor-only attention mask of the
// flattened token tree and the position of every node (spec_origins, SpecInfer)
//
// Row i starts as {i, parent(i)} and its jump pointer as the grandparent; each round ORs
// in the row of the node the pointer names and doubles the pointer, so after r rounds
// the row holds every ancestor within 2^(r+1) steps.  Rows only ever gain true ancestors,
// so a row read while its owner updates it in the same round is still a subset of the
// answer.  The rows live in LDS when they fit, otherwise in the output itself.

constexpr int kMaskLdsWords = 8192;  // N * W words kept in LDS (N <= 512)

struct MaskSmem {
    int par[SPEC_MAX_N];
    int anc[SPEC_MAX_N];
    int dep[SPEC_MAX_N];
    int jmp[SPEC_MAX_N];
    uint32_t rows[kMaskLdsWords];
};

__global__ __launch_bounds__(kBlock) void k_tree_mask(const int32_t* parents,
                                                      const int32_t* base_pos, int N,
                                                      uint32_t* mask, int32_t* positions) {
    __shared__ MaskSmem sm;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int W = (N + 31) / 32;
    const int32_t* par_g = parents + (size_t)b * N;
    uint32_t* out = mask + (size_t)b * N * W;
    bool bad = false;
    for (int i = tid; i < N; i += kBlock) {
        const int p = par_g[i];
        sm.par[i] = p;
        if (i == 0 ? p != -1 : (p < 0 || p >= i)) bad = true;
    }
    bad = __syncthreads_or(bad);
    if (bad) {
        for (int e = tid; e < N * W; e += kBlock) out[e] = 0u;
        if (positions)
            for (int i = tid; i < N; i += kBlock) positions[(size_t)b * N + i] = -1;
        return;
    }
    uint32_t* rows = N * W <= kMaskLdsWords ? sm.rows : out;
    for (int e = tid; e < N * W; e += kBlock) {
        const int i = e / W, w = e - i * W;
        const int p = sm.par[i];
        uint32_t bits = (i >> 5) == w ? 1u << (i & 31) : 0u;
        if (p >= 0 && (p >> 5) == w) bits |= 1u << (p & 31);
        rows[e] = bits;
    }
    for (int i = tid; i < N; i += kBlock) {
        const int p = sm.par[i];
        sm.jmp[i] = p >= 0 ? sm.par[p] : -1;
    }
    bool more = true;
    while (__syncthreads_or(more)) {
        for (int e = tid; e < N * W; e += kBlock) {
            const int i = e / W, w = e - i * W;
            const int j = sm.jmp[i];
            if (j >= 0) rows[e] |= rows[j * W + w];
        }
        __syncthreads();
        int nj[SPEC_MAX_N / kBlock];
        int c = 0;
        for (int i = tid; i < N; i += kBlock, ++c) {
            const int j = sm.jmp[i];
            nj[c] = j >= 0 ? sm.jmp[j] : -1;
        }
        __syncthreads();
        more = false;
        c = 0;
        for (int i = tid; i < N; i += kBlock, ++c) {
            sm.jmp[i] = nj[c];
            more = more || nj[c] >= 0;
        }
    }
    if (rows != out)
        for (int e = tid; e < N * W; e += kBlock) out[e] = rows[e];
    if (positions) {
        tree_depths(sm.par, N, sm.anc, sm.dep);
        const int base = base_pos ? base_pos[b] : 0;
        for (int i = tid; i < N; i += kBlock) positions[(size_t)b * N + i] = base + sm.dep[i];
    }
}

// ---------------------------------------------------------------------------------------
// k_commit_kv: commits the accepted path of a token tree -- output row d of a request is
// the KV row of the d-th node of the path (the root first); one workgroup per (request,
// output row, chunk of kCommitChunk bytes), so every row is copied by independent,
// coalesced 16-byte loads and stores.

constexpr int kCommitChunk = 4 * 16 * kBlock;  // 16 KB per workgroup

__global__ __launch_bounds__(kBlock) void k_commit_kv(const int32_t* accepted_nodes,
                                                      const int32_t* accept_len, int D, int N,
                                                      const uint8_t* kv_tree, uint8_t* kv_out,
                                                      size_t row_bytes, int nchunks,
                                                      int32_t* slots, int vec) {
    __shared__ int node_sm;
    const int tid = threadIdx.x;
    const int blk = blockIdx.x;
    const int c = blk % nchunks;
    const int d = (blk / nchunks) % (D + 1);
    const int b = blk / nchunks / (D + 1);
    if (tid == 0) {
        const int32_t* nodes = accepted_nodes + (size_t)b * D;
        const int k = accept_len[b];
        bool valid = k >= 0 && k <= D;
        for (int e = 0; e < k && valid; ++e)
            if (nodes[e] < 0 || nodes[e] >= N) valid = false;
        int node = -1;
        if (valid && d <= k) node = d == 0 ? 0 : nodes[d - 1];
        if (slots && c == 0) slots[(size_t)b * (D + 1) + d] = node;
        node_sm = node;
    }
    __syncthreads();
    const int node = node_sm;
    if (node < 0) return;
    const uint8_t* src = kv_tree + ((size_t)b * N + node) * row_bytes;
    uint8_t* dst = kv_out + ((size_t)b * (D + 1) + d) * row_bytes;
    const size_t c0 = (size_t)c * kCommitChunk;
    const size_t c1 = c0 + kCommitChunk < row_bytes ? c0 + kCommitChunk : row_bytes;
    if (vec) {  // row_bytes and both bases 16-byte aligned
        const u32x4* s4 = reinterpret_cast<const u32x4*>(src + c0);
        u32x4* d4 = reinterpret_cast<u32x4*>(dst + c0);
        const int nv = (int)((c1 - c0) / 16);
        u32x4 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (u * kBlock + tid < nv) r[u] = ld_stream(s4 + u * kBlock + tid);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (u * kBlock + tid < nv) d4[u * kBlock + tid] = r[u];
    } else {
        for (size_t e = c0 + tid; e < c1; e += kBlock) dst[e] = src[e];
    }
}

// ---------------------------------------------------------------------------------------
// host side

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The walks' call counter (first 256 bytes), then one exit word per request.
constexpr size_t kHeaderBytes = 256 + 4 * (size_t)kExitWords;
static_assert(kHeaderBytes % 256 == 0, "the header keeps the regions after it aligned");

struct Layout {
    size_t parts, dstate, mass, massfb, seg, excl, frows, kept, xch, total;
};

// Workgroups per request that the tree walks may use (the hand-off slots are sized for it).
inline int tree_cluster_max(int B) {
    return B <= 0 ? 1 : std::max(1, std::min(kMaxCluster, 2048 / B));
}

// 64-bit hand-off words per request: at most 2N steps (a row pass per reached node and a
// residual pass per rejected child), W workgroups, three words each.
inline size_t cluster_stride(int N, int W) { return (size_t)2 * N * W * 3; }

inline long fine_chunks(int V) { return ((long)V + kFine - 1) / kFine; }

// Records are stored with a row stride of S (the split count of the call), but the
// workspace is sized for the largest split count so that its size depends only on
// op, B, R and V.
Layout layout_for(int op, int B, int R, int V) {
    Layout L;
    const size_t S2 = (size_t)fine_chunks(V);
    size_t off = kHeaderBytes;  // the header: the walks' call counter and exit words
    L.parts = off;
    if (op != SPEC_OP_TREE_MSS) off = align256(off + sizeof(Part) * (size_t)B * R * kMaxSplits);
    L.dstate = off;
    off = align256(off + sizeof(DrawState) * (size_t)B);
    L.mass = off;
    off = align256(off + sizeof(double) * (size_t)B * S2);
    L.massfb = off;
    off = align256(off + sizeof(double) * (size_t)B * S2);
    L.seg = off;
    off = align256(off + sizeof(double) * (size_t)B * S2 * kSegs);
    L.excl = off;
    if (op == SPEC_OP_TREE) off = align256(off + sizeof(int32_t) * (size_t)B * SPEC_MAX_N);
    L.frows = off;
    if (op == SPEC_OP_CHAIN_FILTERED) off = align256(off + sizeof(FiltRow) * (size_t)B * (2 * R - 1));
    L.kept = off;
    if (op == SPEC_OP_CHAIN_FILTERED) off = align256(off + sizeof(int32_t) * (size_t)B * R * (kBlock + 1));
    L.xch = off;
    if (op == SPEC_OP_GREEDY)
        off = align256(off + sizeof(unsigned long long) * (size_t)B * R * kMaxCluster * 3);
    else if (op == SPEC_OP_CHAIN)  // a step per position, then the draw's slice totals (2)
        off = align256(off + sizeof(unsigned long long) * (size_t)B * (R + 2) * kMaxCluster * 3);
    else if (op == SPEC_OP_TREE)  // at most one step per node
        off = align256(off + sizeof(unsigned long long) * (size_t)B * R * tree_cluster_max(B) * 3);
    else if (op == SPEC_OP_TREE_MSS)
        off = align256(off + sizeof(unsigned long long) * (size_t)B * cluster_stride(R, tree_cluster_max(B)));
    L.total = off;
    return L;
}

void bind_workspace(KArgs& a, void* ws, int op) {
    const Layout L = layout_for(op, a.B, a.R, a.V);
    char* base = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<unsigned*>(base);
    a.parts = reinterpret_cast<Part*>(base + L.parts);
    a.dstate = reinterpret_cast<DrawState*>(base + L.dstate);
    a.mass = reinterpret_cast<double*>(base + L.mass);
    a.massfb = reinterpret_cast<double*>(base + L.massfb);
    a.seg = reinterpret_cast<double*>(base + L.seg);
    a.excl = op == SPEC_OP_TREE ? reinterpret_cast<int32_t*>(base + L.excl) : nullptr;
    a.frows = op == SPEC_OP_CHAIN_FILTERED ? reinterpret_cast<FiltRow*>(base + L.frows) : nullptr;
    a.kept = op == SPEC_OP_CHAIN_FILTERED ? reinterpret_cast<int32_t*>(base + L.kept) : nullptr;
}

// Split each row into S chunks of `chunk` elements (a multiple of 8): about 64 KB of
// logits per workgroup, at least ~2048 workgroups in flight, and at least 1024
// elements per chunk.  `want` > 0 (spec_options.splits) sets the count instead.
void choose_split(long rows, int V, int esize, int want, int* S_out, int* chunk_out) {
    const long row_bytes = (long)V * esize;
    long s = (row_bytes + kChunkBytes - 1) / kChunkBytes;
    const long min_wgs = 2048;
    if (rows * s < min_wgs) s = (min_wgs + rows - 1) / rows;
    const long by_size = V / 1024 > 1 ? V / 1024 : 1;
    if (s > by_size) s = by_size;
    if (want >= 1) s = want;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < 1) s = 1;
    long ch = ((long)V + s - 1) / s;
    ch = (ch + 7) / 8 * 8;
    s = ((long)V + ch - 1) / ch;
    *S_out = (int)s;
    *chunk_out = (int)ch;
}

// Launch options with every field the library chooses filled in.
struct Opts {
    bool eager;
    int cluster;    // 0: from the occupancy
    int splits;     // 0: from the row size
    bool cached;    // chain walk: cache-allocating row loads
    int spin;
};

Opts resolve(const spec_options* o) {
    Opts r;
    r.eager = o && o->path == SPEC_PATH_EAGER;
    r.cluster = o && o->cluster > 0 ? o->cluster : 0;
    r.splits = o && o->splits > 0 ? o->splits : 0;
    r.cached = !(o && o->row_loads == SPEC_LOADS_STREAMING);
    r.spin = o && o->spin_limit > 0 ? o->spin_limit : kSpinMax;
    return r;
}

int check_opts(const spec_options* o) {
    if (!o) return SPEC_OK;
    if (o->path != SPEC_PATH_WALK && o->path != SPEC_PATH_EAGER) return SPEC_ERR_PARAM;
    if (o->row_loads < SPEC_LOADS_DEFAULT || o->row_loads > SPEC_LOADS_STREAMING) return SPEC_ERR_PARAM;
    if (o->cluster < 0 || o->splits < 0 || o->spin_limit < 0) return SPEC_ERR_PARAM;
    return SPEC_OK;
}

// Launch shapes of a call; SPEC_ERR_SHAPE when a grid would exceed 2^32 work-items.
int setup_shapes(KArgs& a, int esize, const Opts& o) {
    choose_split((long)a.B * a.R, a.V, esize, o.splits, &a.S, &a.chunk);
    a.S2 = (int)fine_chunks(a.V);
    const long long lim = 0xffffffffLL / kBlock;
    if ((long long)a.B * a.R * a.S > lim || (long long)a.B * a.S2 > lim) return SPEC_ERR_SHAPE;
    return SPEC_OK;
}

int check_common(const void* logits, int dtype, int B, int V, void* ws, size_t ws_bytes,
                 int op, int R) {
    if (!logits || (B > 0 && !ws)) return SPEC_ERR_NULL;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    if (B < 0 || V < 1) return SPEC_ERR_SHAPE;
    const size_t es = dtype == SPEC_F32 ? 4 : 2;
    // a row's bytes fit a 32-bit signed offset (the row passes' buffer loads)
    if ((long long)V * (long long)es > (long long)INT_MAX) return SPEC_ERR_SHAPE;
    if (((uintptr_t)logits) % es) return SPEC_ERR_PARAM;
    if ((long long)B * R * kMaxSplits > (long long)INT_MAX) return SPEC_ERR_SHAPE;
    if (B > 0) {
        if (((uintptr_t)ws) % 256) return SPEC_ERR_WORKSPACE;
        if (ws_bytes < spec_workspace_bytes(op, B, R, V)) return SPEC_ERR_WORKSPACE;
    }
    return SPEC_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP; }

// Workgroups of `kernel` (kBlock threads) that the current device holds at once: `all`
// counts what the occupancy query allows, `walk` at most kWalkPerCu per compute unit.
// Above five per CU the walks slowed down on the large batch (greedy 52 -> 55-62 us,
// chain 101 -> 118-124 us at six to eight), although the occupancy query allows seven
// (greedy) or five (chain): the later workgroups then start only as earlier ones finish,
// and their clusters wait for them.  The figures are cached per (kernel, device); a
// cached value is written whole by whichever thread gets there first, and every thread
// computes the same one, so concurrent first calls agree.
constexpr int kWalkPerCu = 5;
struct Resident {
    int all, walk;
};
// one cache slot per (kernel, dtype): greedy walk 0/1, chain walk 2/3, tree walk 4/5,
// multi-step tree walk 6/7 (fp32 / bf16)
constexpr int kResidentSlots = 8;
inline Resident resident_blocks(const void* kernel, int slot) {
    static std::atomic<long long> cache[kResidentSlots][64];  // 0: not known; else (all << 32) | walk
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || slot < 0 ||
        slot >= kResidentSlots)
        return {0, 0};
    long long v = cache[slot][dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, nb = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kBlock, 0) != hipSuccess)
            nb = 0;
        // The query can count more workgroups than the compute unit holds: LDS is allocated
        // in granules of 1280 bytes (a co-residency probe ran four 40 KB workgroups per CU
        // at once, but not five of exactly 32 KB, which the query allows), so the LDS
        // bound is taken again with that granule.
        hipFuncAttributes fa;
        int lds_cu = 0;
        if (nb > 0 && hipFuncGetAttributes(&fa, kernel) == hipSuccess &&
            hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) == hipSuccess &&
            fa.sharedSizeBytes > 0 && lds_cu > 0) {
            constexpr size_t kLdsGranule = 1280;
            const size_t per = (fa.sharedSizeBytes + kLdsGranule - 1) / kLdsGranule * kLdsGranule;
            nb = std::min(nb, (int)((size_t)lds_cu / per));
        }
        const long long all = (long long)std::max(0, nb) * std::max(0, cus);
        const long long walk = (long long)std::min(std::max(0, nb), kWalkPerCu) * std::max(0, cus);
        v = (all << 32) | walk | (1LL << 62);  // bit 62: known (a zero device count stays known)
        cache[slot][dev].store(v, std::memory_order_relaxed);
    }
    return {(int)((v >> 32) & 0x3fffffff), (int)(v & 0xffffffff)};
}

// Cluster shape of a position-by-position walk: W workgroups per request, each owning
// `per_chunks` whole fine chunks of every row, with all B * W workgroups resident at once.
// A requested width (spec_options.cluster) is clamped to what the device holds for the
// batch.  A batch too large for the exit words walks with W = 1 (no hand-offs).
inline void walk_shape(const KArgs& a, Resident cap, int want, int* W_out, int* per_chunks_out) {
    int W = std::min(kMaxCluster, std::max(1, cap.walk / std::max(1, a.B)));
    if (want > 0) W = std::max(1, std::min({kMaxCluster, want, cap.all / std::max(1, a.B)}));
    if (a.B > kExitWords) W = 1;
    W = std::min(W, a.S2);
    const int per_chunks = (a.S2 + W - 1) / W;
    *W_out = (a.S2 + per_chunks - 1) / per_chunks;
    *per_chunks_out = per_chunks;
}

template <typename T>
int run_greedy_walk(KArgs& a, unsigned long long* xslots, const Opts& o, hipStream_t st) {
    int W, per;
    walk_shape(a, resident_blocks(reinterpret_cast<const void*>(&k_greedy_walk<T>),
                                  sizeof(T) == 4 ? 0 : 1), o.cluster, &W, &per);
    hipLaunchKernelGGL((k_greedy_walk<T>), dim3(a.B * W), dim3(kBlock), 0, st, a, W,
                       per * kFine, a.hdr, W > 1 ? xslots : (unsigned long long*)nullptr,
                       a.R * W * 3);
    return launch_status();
}

template <typename T>
int run_chain_walk(KArgs& a, unsigned long long* xslots, const Opts& o, hipStream_t st) {
    // cache-allocating row loads keep the slice of the row drawn from near for the final
    // weights (the default)
    a.walk_temporal = o.cached ? 1 : 0;
    int W, per;
    walk_shape(a, resident_blocks(reinterpret_cast<const void*>(&k_chain_walk<T>),
                                  sizeof(T) == 4 ? 2 : 3), o.cluster, &W, &per);
    a.walk_draw = per <= 64 ? 1 : 0;  // a slice's chunk masses fit one wave: draw in the walk
    // hand-off steps: one per position, then the slice totals (and their fallback)
    hipLaunchKernelGGL((k_chain_walk<T>), dim3(a.B * W), dim3(kBlock), 0, st, a, W,
                       per * kFine, a.hdr, W > 1 ? xslots : (unsigned long long*)nullptr,
                       (a.R + 2) * W * 3);
    int rc = launch_status();
    if (rc != SPEC_OK || a.walk_draw) return rc;
    hipLaunchKernelGGL((k_draw<T, false>), dim3(a.B), dim3(64), 0, st, a);
    return launch_status();
}

// The eager passes (every row streamed, then merged) instead of the walks: selected with
// spec_options.path = SPEC_PATH_EAGER.
template <typename T>
int run_greedy(KArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_rows<T, false>), dim3(a.B * a.R * a.S), dim3(kBlock), 0, st, a);
    int rc = launch_status();
    if (rc != SPEC_OK) return rc;
    hipLaunchKernelGGL((k_greedy_merge<T>), dim3(a.B), dim3(kBlock), 0, st, a);
    return launch_status();
}

template <typename T, bool kFilt = false>
int run_draw(KArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_mass<T, kFilt>), dim3(a.B * a.S2), dim3(kBlock), 0, st, a);
    int rc = launch_status();
    if (rc != SPEC_OK) return rc;
    hipLaunchKernelGGL((k_draw<T, kFilt>), dim3(a.B), dim3(64), 0, st, a);
    return launch_status();
}

template <typename T>
int run_chain(KArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_rows<T, true>), dim3(a.B * a.R * a.S), dim3(kBlock), 0, st, a);
    int rc = launch_status();
    if (rc != SPEC_OK) return rc;
    hipLaunchKernelGGL((k_chain_accept<T>), dim3(a.B), dim3(kBlock), 0, st, a);
    rc = launch_status();
    if (rc != SPEC_OK) return rc;
    return run_draw<T>(a, st);
}

template <typename T>
int run_tree_walk(KArgs& a, int sampling, unsigned long long* xslots, const Opts& o,
                  hipStream_t st) {
    int W, per;
    walk_shape(a, resident_blocks(reinterpret_cast<const void*>(&k_tree_walk<T>),
                                  sizeof(T) == 4 ? 4 : 5), o.cluster, &W, &per);
    W = std::min(W, tree_cluster_max(a.B));
    per = (a.S2 + W - 1) / W;
    W = (a.S2 + per - 1) / per;
    hipLaunchKernelGGL((k_tree_walk<T>), dim3(a.B * W), dim3(kBlock), 0, st, a, sampling, W,
                       per * kFine, a.hdr, W > 1 ? xslots : (unsigned long long*)nullptr,
                       a.R * W * 3);
    int rc = launch_status();
    if (rc != SPEC_OK || !sampling) return rc;
    hipLaunchKernelGGL((k_draw<T, false>), dim3(a.B), dim3(64), 0, st, a);
    return launch_status();
}

template <typename T>
int run_tree(KArgs& a, int sampling, hipStream_t st) {
    if (sampling)
        hipLaunchKernelGGL((k_rows<T, true>), dim3(a.B * a.R * a.S), dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((k_rows<T, false>), dim3(a.B * a.R * a.S), dim3(kBlock), 0, st, a);
    int rc = launch_status();
    if (rc != SPEC_OK) return rc;
    hipLaunchKernelGGL((k_tree<T>), dim3(a.B), dim3(kBlock), 0, st, a, sampling);
    rc = launch_status();
    if (rc != SPEC_OK || !sampling) return rc;
    return run_draw<T>(a, st);
}

template <typename T>
int run_tree_mss(KArgs& a, unsigned long long* xslots, const Opts& o, hipStream_t st) {
    int W, per;
    walk_shape(a, resident_blocks(reinterpret_cast<const void*>(&k_mss_walk<T>),
                                  sizeof(T) == 4 ? 6 : 7), o.cluster, &W, &per);
    W = std::min(W, tree_cluster_max(a.B));
    per = (a.S2 + W - 1) / W;
    W = (a.S2 + per - 1) / per;
    hipLaunchKernelGGL((k_mss_walk<T>), dim3(a.B * W), dim3(kBlock), 0, st, a, W, per * kFine,
                       a.hdr, W > 1 ? xslots : (unsigned long long*)nullptr,
                       (int)cluster_stride(a.R, W));
    int rc = launch_status();
    if (rc != SPEC_OK) return rc;
    hipLaunchKernelGGL((k_draw<T, false>), dim3(a.B), dim3(64), 0, st, a);
    return launch_status();
}

template <typename T>
int run_chain_filtered(KArgs& a, hipStream_t st) {
    const int G = a.R - 1;
    hipLaunchKernelGGL((k_filter_rows<T>), dim3(a.B * (a.R + G)), dim3(kBlock), 0, st, a);
    int rc = launch_status();
    if (rc != SPEC_OK) return rc;
    hipLaunchKernelGGL((k_filter_accept<T>), dim3(a.B), dim3(kBlock), 0, st, a);
    rc = launch_status();
    if (rc != SPEC_OK) return rc;
    return run_draw<T, true>(a, st);
}

// ---------------------------------------------------------------------------------------
// measurement utilities: the read ceiling and the exponential throughput of this device

// Each workgroup streams kCalibChunk bytes (the last one the rest) with 16-byte
// non-temporal loads, 8 in flight per lane, and folds them into one value; the sink is
// written only if that value equals a sentinel, so no load can be dropped.
constexpr size_t kCalibChunk = 256 * 1024;
__global__ __launch_bounds__(kBlock) void k_calib_read(const u32x4* data, size_t nvec,
                                                      float* sink) {
    const size_t v0 = (size_t)blockIdx.x * (kCalibChunk / 16);
    const size_t v1 = min(nvec, v0 + kCalibChunk / 16);
    uint32_t acc = 0u;
    size_t v = v0 + threadIdx.x;
    for (; v + 7 * kBlock < v1; v += 8 * kBlock) {
        u32x4 r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) r[u] = ld_stream(data + v + u * kBlock);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
    }
    for (; v < v1; v += kBlock) {
        const u32x4 r = ld_stream(data + v);
        acc ^= r.x ^ r.y ^ r.z ^ r.w;
    }
    if (acc == 0x7fc0deadu) sink[0] = __uint_as_float(acc);
}

// Eight independent exponential chains per lane; the sink is written only on a sentinel.
__global__ __launch_bounds__(kBlock) void k_calib_exp(int iters, float* sink) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = -0.001f * (float)(threadIdx.x + e);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ex2(x[e]) - 1.0f;
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[e];
    if (s == 12345.5f) sink[0] = s;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// The static scratch of spec_verify_chain_noalloc: a chain call's workspace in the
// library's own device memory, zero at load.  Each device holds its own copy until the
// process ends.  Host code never uses this name as an address (on the host it stands for
// a host-side shadow): the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// The device address of `scratch` on the current device (nullptr if HIP cannot give it).
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

// ---------------------------------------------------------------------------------------
// C ABI

extern "C" size_t spec_workspace_bytes(int op, int B, int R, int V) {
    if (B < 0 || R < 1 || V < 1) return 0;
    if (op == SPEC_OP_GREEDY || op == SPEC_OP_CHAIN || op == SPEC_OP_CHAIN_FILTERED) {
        if (R - 1 < 1 || R - 1 > SPEC_MAX_G) return 0;
    } else if (op == SPEC_OP_TREE || op == SPEC_OP_TREE_MSS) {
        if (R > SPEC_MAX_N) return 0;
    } else {
        return 0;
    }
    return layout_for(op, B, R, V).total;
}

extern "C" const char* spec_status_str(int status) {
    switch (status) {
        case SPEC_OK: return "ok";
        case SPEC_ERR_NULL: return "required pointer is NULL";
        case SPEC_ERR_SHAPE: return "size outside the supported range";
        case SPEC_ERR_DTYPE: return "unknown logit dtype";
        case SPEC_ERR_PARAM: return "bad mode, threshold or pointer alignment";
        case SPEC_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
        case SPEC_ERR_HIP: return "HIP launch failed";
        case SPEC_ERR_TOO_LARGE:
            return "the call needs more scratch than the library's static 32 MiB holds";
        default: return "unknown status";
    }
}

extern "C" int spec_verify_greedy_opt(const void* logits, int dtype,
                                      const int32_t* draft_tokens, int B, int G, int V,
                                      int32_t* accept_len, int32_t* out_tokens, void* workspace,
                                      size_t ws_bytes, void* stream, const spec_options* opt) {
    if (!draft_tokens || !accept_len || !out_tokens) return SPEC_ERR_NULL;
    if (G < 1 || G > SPEC_MAX_G) return SPEC_ERR_SHAPE;
    int rc = check_common(logits, dtype, B, V, workspace, ws_bytes, SPEC_OP_GREEDY, G + 1);
    if (rc == SPEC_OK) rc = check_opts(opt);
    if (rc != SPEC_OK || B == 0) return rc;
    const Opts o = resolve(opt);
    KArgs a = {};
    a.logits = logits;
    a.tokens = draft_tokens;
    a.B = B;
    a.R = G + 1;
    a.V = V;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.spin = o.spin;
    rc = setup_shapes(a, dtype == SPEC_F32 ? 4 : 2, o);
    if (rc != SPEC_OK) return rc;
    bind_workspace(a, workspace, SPEC_OP_GREEDY);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!o.eager) {
        const Layout L = layout_for(SPEC_OP_GREEDY, B, G + 1, V);
        unsigned long long* xs =
            reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + L.xch);
        return dtype == SPEC_F32 ? run_greedy_walk<float>(a, xs, o, st)
                                 : run_greedy_walk<uint16_t>(a, xs, o, st);
    }
    return dtype == SPEC_F32 ? run_greedy<float>(a, st) : run_greedy<uint16_t>(a, st);
}

extern "C" int spec_verify_greedy(const void* logits, int dtype, const int32_t* draft_tokens,
                                  int B, int G, int V, int32_t* accept_len, int32_t* out_tokens,
                                  void* workspace, size_t ws_bytes, void* stream) {
    return spec_verify_greedy_opt(logits, dtype, draft_tokens, B, G, V, accept_len, out_tokens,
                                  workspace, ws_bytes, stream, nullptr);
}

extern "C" int spec_verify_chain_opt(const void* logits, int dtype, const float* draft_probs,
                                     const int32_t* draft_tokens, const float* coins,
                                     const float* temperature, int B, int G, int V,
                                     int32_t* accept_len, int32_t* out_tokens, float* probs_out,
                                     void* workspace, size_t ws_bytes, void* stream,
                                     const spec_options* opt) {
    if (!draft_probs || !draft_tokens || !coins || !temperature || !accept_len || !out_tokens)
        return SPEC_ERR_NULL;
    if (G < 1 || G > SPEC_MAX_G) return SPEC_ERR_SHAPE;
    int rc = check_common(logits, dtype, B, V, workspace, ws_bytes, SPEC_OP_CHAIN, G + 1);
    if (rc == SPEC_OK) rc = check_opts(opt);
    if (rc != SPEC_OK || B == 0) return rc;
    const Opts o = resolve(opt);
    if (((uintptr_t)draft_probs) % 4) return SPEC_ERR_PARAM;
    KArgs a = {};
    a.logits = logits;
    a.q = draft_probs;
    a.tokens = draft_tokens;
    a.coins = coins;
    a.coin_stride = G + 1;  // [B][G + 1] coins, the last one for the final draw
    a.temperature = temperature;
    a.B = B;
    a.R = G + 1;
    a.V = V;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.probs = probs_out;
    a.spin = o.spin;
    rc = setup_shapes(a, dtype == SPEC_F32 ? 4 : 2, o);
    if (rc != SPEC_OK) return rc;
    bind_workspace(a, workspace, SPEC_OP_CHAIN);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!o.eager) {
        const Layout L = layout_for(SPEC_OP_CHAIN, B, G + 1, V);
        unsigned long long* xs =
            reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + L.xch);
        return dtype == SPEC_F32 ? run_chain_walk<float>(a, xs, o, st)
                                 : run_chain_walk<uint16_t>(a, xs, o, st);
    }
    return dtype == SPEC_F32 ? run_chain<float>(a, st) : run_chain<uint16_t>(a, st);
}

extern "C" int spec_verify_chain(const void* logits, int dtype, const float* draft_probs,
                                 const int32_t* draft_tokens, const float* coins,
                                 const float* temperature, int B, int G, int V,
                                 int32_t* accept_len, int32_t* out_tokens, float* probs_out,
                                 void* workspace, size_t ws_bytes, void* stream) {
    return spec_verify_chain_opt(logits, dtype, draft_probs, draft_tokens, coins, temperature, B,
                                 G, V, accept_len, out_tokens, probs_out, workspace, ws_bytes,
                                 stream, nullptr);
}

extern "C" int spec_verify_chain_noalloc(const void* logits, int dtype, const float* draft_probs,
                                         const int32_t* draft_tokens, const float* coins,
                                         const float* temperature, int B, int G, int V,
                                         int32_t* accept_len, int32_t* out_tokens,
                                         float* probs_out, void* stream) {
    // every argument check first (as a call with no requests, which enqueues nothing)
    int rc = spec_verify_chain_opt(logits, dtype, draft_probs, draft_tokens, coins, temperature,
                                   0, G, V, accept_len, out_tokens, probs_out, nullptr, 0, stream,
                                   nullptr);
    if (rc != SPEC_OK) return rc;
    if (B < 0) return SPEC_ERR_SHAPE;
    if (B == 0) return SPEC_OK;
    const size_t need = spec_workspace_bytes(SPEC_OP_CHAIN, B, G + 1, V);
    if (need == 0) return SPEC_ERR_SHAPE;
    if (need > kScratchBytes) return SPEC_ERR_TOO_LARGE;
    void* ws = scratch_ptr();
    if (!ws) return SPEC_ERR_HIP;
    return spec_verify_chain_opt(logits, dtype, draft_probs, draft_tokens, coins, temperature, B,
                                 G, V, accept_len, out_tokens, probs_out, ws, kScratchBytes,
                                 stream, nullptr);
}

extern "C" int spec_verify_tree_opt(const void* logits, int dtype, const int32_t* node_tokens,
                                    const int32_t* parents, const float* coins,
                                    const float* temperature, int B, int N, int V, int D,
                                    int mode, float threshold_single, float threshold_acc,
                                    int32_t* accept_len, int32_t* out_tokens,
                                    int32_t* accepted_nodes, float* probs_out, void* workspace,
                                    size_t ws_bytes, void* stream, const spec_options* opt) {
    if (!node_tokens || !parents || !accept_len || !out_tokens || !accepted_nodes)
        return SPEC_ERR_NULL;
    if (mode != SPEC_TREE_GREEDY && mode != SPEC_TREE_SAMPLING) return SPEC_ERR_PARAM;
    if (mode == SPEC_TREE_SAMPLING) {
        if (!coins || !temperature) return SPEC_ERR_NULL;
        if (!(threshold_single > 0.f) || !(threshold_acc > 0.f)) return SPEC_ERR_PARAM;
    }
    if (N < 1 || N > SPEC_MAX_N || D < 1 || D > SPEC_MAX_N) return SPEC_ERR_SHAPE;
    int rc = check_common(logits, dtype, B, V, workspace, ws_bytes, SPEC_OP_TREE, N);
    if (rc == SPEC_OK) rc = check_opts(opt);
    if (rc != SPEC_OK || B == 0) return rc;
    const Opts o = resolve(opt);
    KArgs a = {};
    a.logits = logits;
    a.tokens = node_tokens;
    a.parents = parents;
    a.coins = coins;
    a.coin_stride = D + 1;  // [B][D + 1] coins, the last one for the final draw
    a.temperature = temperature;
    a.B = B;
    a.R = N;
    a.V = V;
    a.D = D;
    a.th_single = threshold_single;
    a.th_acc = threshold_acc;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.accepted_nodes = accepted_nodes;
    a.probs = probs_out;
    a.spin = o.spin;
    rc = setup_shapes(a, dtype == SPEC_F32 ? 4 : 2, o);
    if (rc != SPEC_OK) return rc;
    bind_workspace(a, workspace, SPEC_OP_TREE);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!o.eager) {
        const Layout L = layout_for(SPEC_OP_TREE, B, N, V);
        unsigned long long* xs =
            reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + L.xch);
        return dtype == SPEC_F32 ? run_tree_walk<float>(a, mode, xs, o, st)
                                 : run_tree_walk<uint16_t>(a, mode, xs, o, st);
    }
    return dtype == SPEC_F32 ? run_tree<float>(a, mode, st) : run_tree<uint16_t>(a, mode, st);
}

extern "C" int spec_verify_tree(const void* logits, int dtype, const int32_t* node_tokens,
                                const int32_t* parents, const float* coins,
                                const float* temperature, int B, int N, int V, int D, int mode,
                                float threshold_single, float threshold_acc,
                                int32_t* accept_len, int32_t* out_tokens,
                                int32_t* accepted_nodes, float* probs_out, void* workspace,
                                size_t ws_bytes, void* stream) {
    return spec_verify_tree_opt(logits, dtype, node_tokens, parents, coins, temperature, B, N, V,
                                D, mode, threshold_single, threshold_acc, accept_len, out_tokens,
                                accepted_nodes, probs_out, workspace, ws_bytes, stream, nullptr);
}

extern "C" int spec_verify_tree_mss_opt(const void* logits, int dtype, const float* draft_probs,
                                        const int32_t* node_tokens, const int32_t* parents,
                                        const float* coins, const float* temperature, int B,
                                        int N, int V, int D, int32_t* accept_len,
                                        int32_t* out_tokens, int32_t* accepted_nodes,
                                        float* probs_out, void* workspace, size_t ws_bytes,
                                        void* stream, const spec_options* opt) {
    if (!draft_probs || !node_tokens || !parents || !coins || !temperature || !accept_len ||
        !out_tokens || !accepted_nodes)
        return SPEC_ERR_NULL;
    if (N < 1 || N > SPEC_MAX_N || D < 1 || D > SPEC_MAX_N) return SPEC_ERR_SHAPE;
    int rc = check_common(logits, dtype, B, V, workspace, ws_bytes, SPEC_OP_TREE_MSS, N);
    if (rc == SPEC_OK) rc = check_opts(opt);
    if (rc != SPEC_OK || B == 0) return rc;
    const Opts o = resolve(opt);
    if (((uintptr_t)draft_probs) % 4) return SPEC_ERR_PARAM;
    KArgs a = {};
    a.logits = logits;
    a.q = draft_probs;
    a.tokens = node_tokens;
    a.parents = parents;
    a.coins = coins;
    a.coin_stride = N;  // [B][N] coins, the last one for the final draw
    a.temperature = temperature;
    a.B = B;
    a.R = N;
    a.V = V;
    a.D = D;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.accepted_nodes = accepted_nodes;
    a.probs = probs_out;
    a.spin = o.spin;
    rc = setup_shapes(a, dtype == SPEC_F32 ? 4 : 2, o);
    if (rc != SPEC_OK) return rc;
    bind_workspace(a, workspace, SPEC_OP_TREE_MSS);
    const Layout L = layout_for(SPEC_OP_TREE_MSS, B, N, V);
    unsigned long long* xslots =
        reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + L.xch);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return dtype == SPEC_F32 ? run_tree_mss<float>(a, xslots, o, st)
                             : run_tree_mss<uint16_t>(a, xslots, o, st);
}

extern "C" int spec_verify_tree_mss(const void* logits, int dtype, const float* draft_probs,
                                    const int32_t* node_tokens, const int32_t* parents,
                                    const float* coins, const float* temperature, int B, int N,
                                    int V, int D, int32_t* accept_len, int32_t* out_tokens,
                                    int32_t* accepted_nodes, float* probs_out, void* workspace,
                                    size_t ws_bytes, void* stream) {
    return spec_verify_tree_mss_opt(logits, dtype, draft_probs, node_tokens, parents, coins,
                                    temperature, B, N, V, D, accept_len, out_tokens,
                                    accepted_nodes, probs_out, workspace, ws_bytes, stream,
                                    nullptr);
}

extern "C" int spec_tree_mask(const int32_t* parents, const int32_t* base_pos, int B, int N,
                              uint32_t* mask, int32_t* positions, void* stream) {
    if (!parents || !mask) return SPEC_ERR_NULL;
    if (B < 0 || N < 1 || N > SPEC_MAX_N) return SPEC_ERR_SHAPE;
    if (B == 0) return SPEC_OK;
    hipLaunchKernelGGL(k_tree_mask, dim3(B), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       parents, base_pos, N, mask, positions);
    return launch_status();
}

extern "C" int spec_tree_commit_kv(const int32_t* accepted_nodes, const int32_t* accept_len,
                                   int B, int D, int N, const void* kv_tree, void* kv_out,
                                   size_t row_bytes, int32_t* slots, void* stream) {
    if (!accepted_nodes || !accept_len || !kv_tree || !kv_out) return SPEC_ERR_NULL;
    if (B < 0 || D < 1 || D > SPEC_MAX_N || N < 1 || N > SPEC_MAX_N || row_bytes < 1)
        return SPEC_ERR_SHAPE;
    if (B == 0) return SPEC_OK;
    const long long nchunks = ((long long)row_bytes + kCommitChunk - 1) / kCommitChunk;
    const long long grid = (long long)B * (D + 1) * nchunks;
    if (grid > 0xffffffffLL / kBlock || nchunks > INT_MAX) return SPEC_ERR_SHAPE;
    const int vec = row_bytes % 16 == 0 && ((uintptr_t)kv_tree) % 16 == 0 &&
                    ((uintptr_t)kv_out) % 16 == 0;
    hipLaunchKernelGGL(k_commit_kv, dim3((unsigned)grid), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), accepted_nodes, accept_len, D, N,
                       static_cast<const uint8_t*>(kv_tree), static_cast<uint8_t*>(kv_out),
                       row_bytes, (int)nchunks, slots, vec);
    return launch_status();
}

extern "C" int spec_verify_chain_filtered(const void* logits, const void* draft_logits, int dtype,
                                          const int32_t* draft_tokens, const float* coins,
                                          const float* temperature, const int32_t* top_k,
                                          const float* top_p, int B, int G, int V,
                                          int32_t* accept_len, int32_t* out_tokens,
                                          float* probs_out, void* workspace, size_t ws_bytes,
                                          void* stream) {
    if (!draft_logits || !draft_tokens || !coins || !temperature || !accept_len || !out_tokens)
        return SPEC_ERR_NULL;
    if (G < 1 || G > SPEC_MAX_G) return SPEC_ERR_SHAPE;
    int rc = check_common(logits, dtype, B, V, workspace, ws_bytes, SPEC_OP_CHAIN_FILTERED, G + 1);
    if (rc != SPEC_OK || B == 0) return rc;
    if (((uintptr_t)draft_logits) % (dtype == SPEC_F32 ? 4 : 2)) return SPEC_ERR_PARAM;
    if ((long long)B * (2 * G + 1) > 0xffffffffLL / kBlock) return SPEC_ERR_SHAPE;
    KArgs a = {};
    a.logits = logits;
    a.dlogits = draft_logits;
    a.tokens = draft_tokens;
    a.coins = coins;
    a.coin_stride = G + 1;  // [B][G + 1] coins, the last one for the final draw
    a.temperature = temperature;
    a.top_k = top_k;
    a.top_p = top_p;
    a.B = B;
    a.R = G + 1;
    a.V = V;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.probs = probs_out;
    int lv = 0;
    while ((1L << lv) < (long)V) ++lv;
    a.fixbits = 62 - lv;
    rc = setup_shapes(a, dtype == SPEC_F32 ? 4 : 2, resolve(nullptr));
    if (rc != SPEC_OK) return rc;
    bind_workspace(a, workspace, SPEC_OP_CHAIN_FILTERED);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return dtype == SPEC_F32 ? run_chain_filtered<float>(a, st) : run_chain_filtered<uint16_t>(a, st);
}

extern "C" int spec_calib_read(const void* data, size_t bytes, float* sink, void* stream) {
    if (bytes == 0) return SPEC_OK;
    if (!data || !sink) return SPEC_ERR_NULL;
    if (((uintptr_t)data) % 16 || bytes % 16) return SPEC_ERR_PARAM;
    const size_t blocks = (bytes + kCalibChunk - 1) / kCalibChunk;
    if (blocks > 0x7fffffffULL) return SPEC_ERR_SHAPE;
    hipLaunchKernelGGL(k_calib_read, dim3((unsigned)blocks), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(data),
                       bytes / 16, sink);
    return launch_status();
}

extern "C" int spec_calib_exp(int blocks, int iters, float* sink, void* stream) {
    if (!sink) return SPEC_ERR_NULL;
    if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 20)) return SPEC_ERR_PARAM;
    hipLaunchKernelGGL(k_calib_exp, dim3(blocks), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    return launch_status();
}
