// spec_verify.hip -- HIP kernels for CDNA4 (gfx950) and the C ABI of the speculative
// decoding verify library (include/spec_verify.h).
//
// Kernels
//   k_rows      streams every target-logit row once from HBM (16-byte vector loads,
//               kUnroll loads in flight per lane), split over `S` workgroups per row.
//               Each workgroup reduces its chunk to one 16-byte record: the chunk max,
//               the lowest index attaining it (greedy) and sum exp((l - m)/T) relative to
//               the chunk max (sampling), accumulated in fp32 per batch and fp64 across
//               batches.  Wave64 butterfly shuffles, then LDS across the 4 waves.
//               For the chain calls the last workgroup of a request to finish (arrival
//               counter per request) merges that request's records in split order and
//               runs the acceptance scan; greedy requests and bonus draws end there.
//   k_residual  chain requests rejected at position k: sum of max(0, p_k - q_k) over each
//               chunk of row k (target row re-read from cache, q row from HBM); the last
//               workgroup of the request locates the chunk holding u * S and scans it.
//   k_tree      one workgroup per request: validates the parent array (pointer jumping
//               for depths), walks the tree level by level from the records, then draws
//               the last token with the tried children removed.
//
// Sources: llm-infra-atlas "Speculative Decoding" section 0 and section 2; ricardokevins
// "Speculative Decoding", correction sampling, Eq. a(x) and Eq. r(x); zdszero
// "spec_origins": Blockwise Parallel Decoding (verify), Speculative Decoding (acceptance
// rule items 1-3), SpecInfer, and "in SGLang" (target-only tree walk).

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "spec_verify.h"

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kUnroll = 4;
constexpr int kMaxSplits = 64;
constexpr int kMaxRows = SPEC_MAX_G + 1;
constexpr float kLog2e = 1.44269504088896340736f;

enum RowMode { kGreedyChain = 0, kSamplingChain = 1, kRowsOnlyGreedy = 2, kRowsOnlySampling = 3 };

// One record per (row, split): chunk max, lowest index attaining it, and the chunk's
// sum of exp2((l - m) * log2(e) / T) relative to that max (sampling only).
struct alignas(16) Part {
    float m;
    int idx;
    double z;
};

// Handed from the acceptance scan to the residual pass of a rejected chain request.
struct alignas(16) ResidState {
    int k;
    float M;     // max of row k
    float s2;    // log2(e) / T
    float invZ;  // 1 / Z rounded to fp32 (residual weights)
    double Z;    // sum exp((l - M) / T) over row k
    double T;
};

struct KArgs {
    const void* logits;
    const float* q;
    const int32_t* tokens;  // chain: draft tokens [B][G]; tree: node tokens [B][N]
    const int32_t* parents;
    const float* coins;
    const float* temperature;
    int B, R, V, S, chunk, D;
    float th_single, th_acc;
    int32_t* accept_len;
    int32_t* out_tokens;
    int32_t* accepted_nodes;
    float* probs;
    uint32_t* ticketA;
    uint32_t* ticketB;
    Part* parts;
    ResidState* state;
    double* resid;
};

// ---------------------------------------------------------------------------------------
// element access

template <typename T>
struct Ld;

template <>
struct Ld<float> {
    static constexpr int kVec = 4;
    __device__ static float one(const float* p) { return *p; }
    __device__ static void unpack(const uint4& v, float* f) {
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
    __device__ static void unpack(const uint4& v, float* f) {
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

// (m, z) with z relative to m: merge two partial softmax sums.
__device__ inline void soft_merge(float& m, double& z, float m2, double z2, float s2) {
    float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    double a = (m == M) ? z : z * (double)ex2((m - M) * s2);
    double c = (m2 == M) ? z2 : z2 * (double)ex2((m2 - M) * s2);
    m = M;
    z = a + c;
}

__device__ inline void wave_soft(float& m, double& z, float s2) {
    for (int o = 32; o > 0; o >>= 1) {
        float m2 = __shfl_xor(m, o);
        double z2 = __shfl_xor(z, o);
        soft_merge(m, z, m2, z2, s2);
    }
}

struct Smem {
    float M[kMaxRows];
    double Z[kMaxRows];
    double p[kMaxRows];
    int arg[kMaxRows];
    int x[kMaxRows];
    float l[kMaxRows];
    float qx[kMaxRows];
    float u[kMaxRows];
    double P[kMaxSplits];   // chunk masses of the row being drawn from
    double f[kMaxSplits];   // chunk scale exp((m_s - M) / T)
    double wtot[kWaves];
    float rm[kWaves];
    double rz[kWaves];
    int ri[kWaves];
    int ex_local[64];
    int n_ex_local;
    int k;
    int sstar;
    int fallback;
    double tau;
    int found;
    int lastthr;
    int result;
    int last;
};

// ---------------------------------------------------------------------------------------
// the row pass of one chunk: per-thread streaming state, then a block reduction

template <typename T, bool kSampling>
struct RowState {
    float m = -INFINITY;
    int idx = INT_MAX;
    double z = 0.0;

    // elements must arrive in ascending index order per thread (greedy keeps the first)
    __device__ void push(float x, int j, float s2) {
        if (kSampling) {
            if (x > m) {
                z *= (double)ex2((m - x) * s2);
                m = x;
            }
            if (m != -INFINITY) z += (double)ex2((x - m) * s2);
        } else if (x > m) {
            m = x;
            idx = j;
        }
    }

    template <int kN>
    __device__ void push_batch(const float* f, const int* vec_base, float s2) {
        float bm = f[0];
#pragma unroll
        for (int e = 1; e < kN; ++e) bm = fmaxf(bm, f[e]);
        if (kSampling) {
            if (bm > m) {
                z *= (double)ex2((m - bm) * s2);
                m = bm;
            }
            if (m != -INFINITY) {
                constexpr int kVec = Ld<T>::kVec;
                float acc = 0.f;
#pragma unroll
                for (int u = 0; u < kN / kVec; ++u) {
                    float e8[kVec];
#pragma unroll
                    for (int e = 0; e < kVec; ++e) e8[e] = ex2((f[u * kVec + e] - m) * s2);
                    float s;
                    if (kVec == 8)
                        s = ((e8[0] + e8[1]) + (e8[2] + e8[3])) + ((e8[4] + e8[5]) + (e8[6] + e8[7]));
                    else
                        s = (e8[0] + e8[1]) + (e8[2] + e8[3]);
                    acc += s;
                }
                z += (double)acc;
            }
        } else if (bm > m) {
            constexpr int kVec = Ld<T>::kVec;
#pragma unroll
            for (int e = 0; e < kN; ++e) {
                if (f[e] == bm) {
                    m = bm;
                    idx = vec_base[e / kVec] + (e % kVec);
                    break;
                }
            }
        }
    }
};

// Reduces chunk [c0, c1) of a row into one record (valid in thread 0).
template <typename T, bool kSampling>
__device__ __attribute__((always_inline)) Part chunk_record(const T* rowp, int c0, int c1, float s2, Smem& sm) {
    constexpr int kVec = Ld<T>::kVec;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    RowState<T, kSampling> st;
    const int n = c1 > c0 ? c1 - c0 : 0;
    const T* p = rowp + c0;
    int head = (int)(((16u - ((uint32_t)(uintptr_t)p & 15u)) & 15u) / sizeof(T));
    if (head > n) head = n;
    const int nv = (n - head) / kVec;
    const int tail0 = head + nv * kVec;
    if (tid < head) st.push(Ld<T>::one(p + tid), c0 + tid, s2);
    const uint4* vp = reinterpret_cast<const uint4*>(p + head);
    const int ebase = c0 + head;
    int v = tid;
    for (; v + (kUnroll - 1) * kBlock < nv; v += kUnroll * kBlock) {
        uint4 raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) raw[u] = vp[v + u * kBlock];
        float f[kUnroll * kVec];
        int vb[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            Ld<T>::unpack(raw[u], f + u * kVec);
            vb[u] = ebase + (v + u * kBlock) * kVec;
        }
        st.template push_batch<kUnroll * kVec>(f, vb, s2);
    }
    for (; v < nv; v += kBlock) {
        uint4 raw = vp[v];
        float f[kVec];
        Ld<T>::unpack(raw, f);
        int vb[1] = {ebase + v * kVec};
        st.template push_batch<kVec>(f, vb, s2);
    }
    if (tail0 + tid < n) st.push(Ld<T>::one(p + tail0 + tid), c0 + tail0 + tid, s2);

    float m = st.m;
    int idx = st.idx;
    double z = st.z;
    if (kSampling)
        wave_soft(m, z, s2);
    else
        wave_argmax(m, idx);
    if (lane == 0) {
        sm.rm[wave] = m;
        sm.ri[wave] = idx;
        sm.rz[wave] = z;
    }
    __syncthreads();
    Part r;
    r.m = sm.rm[0];
    r.idx = sm.ri[0];
    r.z = sm.rz[0];
    for (int w = 1; w < kWaves; ++w) {
        if (kSampling)
            soft_merge(r.m, r.z, sm.rm[w], sm.rz[w], s2);
        else
            arg_merge(r.m, r.idx, sm.rm[w], sm.ri[w]);
    }
    return r;
}

// ---------------------------------------------------------------------------------------
// block helpers for the final draw

__device__ inline double block_excl_scan(double v, Smem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double x = v;
    for (int o = 1; o < 64; o <<= 1) {
        double y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    double ex = __shfl_up(x, 1);
    if (lane == 0) ex = 0.0;
    if (lane == 63) sm.wtot[wave] = x;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += sm.wtot[w];
    __syncthreads();
    return off + ex;
}

// First j in [c0, c1) with w(j) > 0 whose inclusive prefix sum (from c0) reaches tau.
// If rounding leaves tau beyond the total, the last j with w(j) > 0.  -1 if none is
// positive.  Every thread of the block must call it; all get the result.
template <typename WF>
__device__ int scan_find(const WF& wf, int c0, int c1, double tau, Smem& sm) {
    const int tid = threadIdx.x;
    const int L = c1 > c0 ? c1 - c0 : 0;
    const int len = (L + kBlock - 1) / kBlock;
    const int j0 = c0 + tid * len;
    const int j1 = min(c1, j0 + len);
    double sum = 0.0;
    int last = -1;
    for (int j = j0; j < j1; ++j) {
        float w = wf(j);
        if (w > 0.f) {
            sum += (double)w;
            last = j;
        }
    }
    double ex = block_excl_scan(sum, sm);
    if (tid == 0) {
        sm.found = INT_MAX;
        sm.lastthr = -1;
        sm.result = -1;
    }
    __syncthreads();
    if (sum > 0.0 && tau <= ex + sum) atomicMin(&sm.found, tid);
    if (sum > 0.0) atomicMax(&sm.lastthr, tid);
    __syncthreads();
    const int found = sm.found;
    const int who = found != INT_MAX ? found : sm.lastthr;
    if (tid == who) {
        int y = last;
        if (found != INT_MAX) {
            double C = ex;
            for (int j = j0; j < j1; ++j) {
                float w = wf(j);
                if (w > 0.f) {
                    C += (double)w;
                    if (tau <= C) {
                        y = j;
                        break;
                    }
                }
            }
        }
        sm.result = y;
    }
    __syncthreads();
    const int y = sm.result;
    __syncthreads();
    return y;
}

template <typename T>
struct RowWeight {  // exp2((l_j - ref) * s2), excluded tokens -> 0
    const T* row;
    float ref, s2;
    const int* ex;
    int nex;
    __device__ float operator()(int j) const {
        for (int e = 0; e < nex; ++e)
            if (ex[e] == j) return 0.f;
        return ex2((Ld<T>::one(row + j) - ref) * s2);
    }
};

template <typename T>
struct ResidualWeight {  // max(0, p_j - q_j) with p_j = exp2((l_j - M) * s2) / Z in fp32
    const T* row;
    const float* q;
    float M, s2, invZ;
    __device__ float operator()(int j) const {
        float p = ex2((Ld<T>::one(row + j) - M) * s2) * invZ;
        return fmaxf(p - q[j], 0.f);
    }
};

// Inverse-CDF draw from the target row (temperature T) with the tokens excl[0..nexcl)
// removed, using the row's split records for the chunk masses.  Falls back to the whole
// row when the remaining mass is not positive.  Block-wide; every thread gets the token.
template <typename T>
__device__ __attribute__((always_inline)) int draw_row(const T* rowp, int V, int chunk, int S, const Part* pr, float M,
                        float s2, double Td, double u, const int* excl, int nexcl, Smem& sm) {
    const int tid = threadIdx.x;
    for (int attempt = 0; attempt < 2; ++attempt) {
        const int nx = attempt == 0 ? nexcl : 0;
        if (tid < S) {
            const float ms = pr[tid].m;
            double zs = pr[tid].z;
            const double fs = ms == -INFINITY ? 0.0 : exp(((double)ms - (double)M) / Td);
            if (nx > 0 && ms != -INFINITY) {
                const int c0 = tid * chunk, c1 = min(V, c0 + chunk);
                double ex = 0.0;
                for (int e = 0; e < nx; ++e) {
                    const int t = excl[e];
                    if (t >= c0 && t < c1) ex += (double)ex2((Ld<T>::one(rowp + t) - ms) * s2);
                }
                if (ex > 0.0) {
                    double rem = zs - ex;
                    zs = rem > zs * 1e-6 ? rem : 0.0;  // below that it is only rounding residue
                }
            }
            sm.P[tid] = zs * fs;
            sm.f[tid] = fs;
        }
        __syncthreads();
        if (tid == 0) {
            double tot = 0.0;
            for (int s = 0; s < S; ++s) tot += sm.P[s];
            sm.fallback = !(tot > 0.0);
            if (!sm.fallback) {
                const double t = u * tot;
                double pre = 0.0, before = 0.0;
                int ss = -1, lastpos = -1;
                for (int s = 0; s < S; ++s) {
                    if (sm.P[s] > 0.0) {
                        lastpos = s;
                        if (t <= pre + sm.P[s]) {
                            ss = s;
                            before = pre;
                            break;
                        }
                    }
                    pre += sm.P[s];
                }
                if (ss < 0) {
                    ss = lastpos;
                    before = pre - sm.P[ss];
                }
                sm.sstar = ss;
                sm.tau = (t - before) / sm.f[ss];
                int nl = 0;
                const int c0 = ss * chunk, c1 = min(V, c0 + chunk);
                for (int e = 0; e < nx; ++e)
                    if (excl[e] >= c0 && excl[e] < c1) {
                        if (nl < 64) sm.ex_local[nl] = excl[e];
                        ++nl;
                    }
                sm.n_ex_local = nl;
            }
        }
        __syncthreads();
        if (sm.fallback) {
            __syncthreads();
            if (nexcl == 0 || attempt == 1) return -1;  // no finite logit at all
            continue;
        }
        const int ss = sm.sstar;
        const bool local = sm.n_ex_local <= 64;
        RowWeight<T> wf{rowp, pr[ss].m, s2, local ? sm.ex_local : excl,
                        local ? sm.n_ex_local : nx};
        const int c0 = ss * chunk, c1 = min(V, c0 + chunk);
        int y = scan_find(wf, c0, c1, sm.tau, sm);
        if (y < 0) y = pr[ss].idx >= 0 && pr[ss].idx < V ? pr[ss].idx : c0;
        return y;
    }
    return -1;
}

// ---------------------------------------------------------------------------------------
// merges run by the last workgroup of a chain request

template <typename T>
__device__ void merge_greedy_chain(const KArgs& a, int b, Smem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = a.R, G = R - 1, S = a.S;
    for (int i = wave; i < R; i += kWaves) {
        const Part* pr = a.parts + ((size_t)b * R + i) * kMaxSplits;
        float v = -INFINITY;
        int ix = INT_MAX;
        if (lane < S) {
            v = pr[lane].m;
            ix = pr[lane].idx;
        }
        wave_argmax(v, ix);
        if (lane == 0) sm.arg[i] = v == -INFINITY ? -1 : ix;
    }
    for (int i = tid; i < G; i += kBlock) sm.x[i] = a.tokens[(size_t)b * G + i];
    __syncthreads();
    if (tid == 0) {
        const int* x = sm.x;
        bool valid = true;
        for (int i = 0; i < G; ++i)
            if (x[i] < 0 || x[i] >= a.V) valid = false;
        for (int i = 0; i < R; ++i)
            if (sm.arg[i] < 0) valid = false;
        int k = G;
        if (valid) {
            for (int i = 0; i < G; ++i)
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

template <typename T>
__device__ void merge_sampling_chain(const KArgs& a, int b, Smem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = a.R, G = R - 1, S = a.S, V = a.V;
    const float Tf = a.temperature[b];
    const bool t_ok = isfinite(Tf) && Tf > 0.f;
    const double Td = (double)Tf;
    const float s2 = kLog2e / Tf;
    for (int i = wave; i < R; i += kWaves) {
        const Part* pr = a.parts + ((size_t)b * R + i) * kMaxSplits;
        float m = -INFINITY;
        double z = 0.0;
        if (lane < S) {
            m = pr[lane].m;
            z = pr[lane].z;
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
    for (int i = tid; i < R; i += kBlock) {
        sm.u[i] = a.coins[(size_t)b * R + i];
        if (i < G) {
            const int xi = a.tokens[(size_t)b * G + i];
            sm.x[i] = xi;
            if (xi >= 0 && xi < V) {
                sm.l[i] = Ld<T>::one(reinterpret_cast<const T*>(a.logits) + ((size_t)b * R + i) * V + xi);
                sm.qx[i] = a.q[((size_t)b * G + i) * V + xi];
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        const int* x = sm.x;
        const float* u = sm.u;
        bool valid = t_ok;
        for (int i = 0; i < G; ++i)
            if (x[i] < 0 || x[i] >= V) valid = false;
        for (int i = 0; i < R; ++i) {
            if (!(u[i] > 0.f && u[i] <= 1.f)) valid = false;
            if (sm.M[i] == -INFINITY) valid = false;
        }
        for (int i = 0; i < G && valid; ++i)
            if (!(sm.qx[i] >= 0.f) || !isfinite(sm.qx[i])) valid = false;
        int k = G;
        if (valid) {
            for (int i = 0; i < G; ++i) {
                const double l = (double)sm.l[i];
                const double p = exp((l - (double)sm.M[i]) / Td) / sm.Z[i];
                const double qx = (double)sm.qx[i];
                const bool accept = qx > 0.0 ? (p > 0.0 && (double)u[i] <= p / qx) : p > 0.0;
                sm.p[i] = p;
                if (!accept) {
                    k = i;
                    break;
                }
            }
        }
        sm.k = valid ? k : -1;
        a.accept_len[b] = sm.k;
        if (valid && k < G) {
            ResidState st;
            st.k = k;
            st.M = sm.M[k];
            st.s2 = s2;
            st.Z = sm.Z[k];
            st.invZ = (float)(1.0 / sm.Z[k]);
            st.T = Td;
            a.state[b] = st;
        }
    }
    __syncthreads();
    const int k = sm.k;
    for (int i = tid; i < R; i += kBlock) {
        int t = -1;
        float pr = 0.f;
        if (k >= 0 && i < k) {
            t = sm.x[i];
            pr = (float)sm.p[i];
        }
        if (i != k) {  // slot k is written by the final draw (bonus here, residual pass later)
            a.out_tokens[(size_t)b * R + i] = t;
            if (a.probs) a.probs[(size_t)b * R + i] = pr;
        }
    }
    if (k != G) return;
    // bonus: every draft accepted, draw from row G
    const T* rowp = reinterpret_cast<const T*>(a.logits) + ((size_t)b * R + G) * V;
    const Part* pr = a.parts + ((size_t)b * R + G) * kMaxSplits;
    const double u = (double)sm.u[G];
    const int y = draw_row<T>(rowp, V, a.chunk, S, pr, sm.M[G], s2, Td, u, nullptr, 0, sm);
    if (tid == 0) {
        a.out_tokens[(size_t)b * R + G] = y;
        if (a.probs) {
            const double l = (double)Ld<T>::one(rowp + y);
            a.probs[(size_t)b * R + G] = (float)(exp((l - (double)sm.M[G]) / Td) / sm.Z[G]);
        }
    }
}

// ---------------------------------------------------------------------------------------
// k_rows: one workgroup per (row, split)

template <typename T, int kMode>
__global__ __launch_bounds__(kBlock) void k_rows(KArgs a) {
    constexpr bool kSampling = kMode == kSamplingChain || kMode == kRowsOnlySampling;
    __shared__ Smem sm;
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
    const Part r = chunk_record<T, kSampling>(rowp, c0, c1, s2, sm);
    if (threadIdx.x == 0) a.parts[(size_t)row * kMaxSplits + s] = r;
    if (kMode == kRowsOnlyGreedy || kMode == kRowsOnlySampling) return;

    // the last workgroup of request b to finish merges its records
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t t = atomicAdd(&a.ticketA[b], 1u);
        sm.last = t == (uint32_t)(a.R * S - 1);
    }
    __syncthreads();
    if (!sm.last) return;
    __threadfence();
    if (threadIdx.x == 0) a.ticketA[b] = 0u;  // every other arrival has happened
    if (kMode == kGreedyChain)
        merge_greedy_chain<T>(a, b, sm);
    else
        merge_sampling_chain<T>(a, b, sm);
}

// ---------------------------------------------------------------------------------------
// k_residual: chain requests rejected at k < G

template <typename T>
__global__ __launch_bounds__(kBlock) void k_residual(KArgs a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = a.S, R = a.R, G = R - 1, V = a.V;
    const int b = blockIdx.x / S;
    const int s = blockIdx.x - b * S;
    const ResidState st = a.state[b];
    const int acc = a.accept_len[b];
    if (acc < 0 || acc >= G) return;  // invalid, or the bonus was already drawn
    const int k = st.k;
    const T* rowp = reinterpret_cast<const T*>(a.logits) + ((size_t)b * R + k) * V;
    const float* qrow = a.q + ((size_t)b * G + k) * V;
    const ResidualWeight<T> wf{rowp, qrow, st.M, st.s2, st.invZ};
    const int c0 = s * a.chunk, c1 = min(V, c0 + a.chunk);

    double sum = 0.0;
    const int n = c1 > c0 ? c1 - c0 : 0;
    const bool aligned = (((uintptr_t)(rowp + c0)) % (4 * sizeof(T)) == 0) &&
                         (((uintptr_t)(qrow + c0)) % 16 == 0);
    int done = 0;
    if (aligned) {
        const int nv = n / 4;
        for (int v = tid; v < nv; v += kBlock) {
            const float4 qv = *reinterpret_cast<const float4*>(qrow + c0 + 4 * v);
            float l[4];
            if (sizeof(T) == 4) {
                const float4 lv = *reinterpret_cast<const float4*>(rowp + c0 + 4 * v);
                l[0] = lv.x; l[1] = lv.y; l[2] = lv.z; l[3] = lv.w;
            } else {
                const uint2 lv = *reinterpret_cast<const uint2*>(rowp + c0 + 4 * v);
                l[0] = __uint_as_float(lv.x << 16);
                l[1] = __uint_as_float(lv.x & 0xffff0000u);
                l[2] = __uint_as_float(lv.y << 16);
                l[3] = __uint_as_float(lv.y & 0xffff0000u);
            }
            const float qq[4] = {qv.x, qv.y, qv.z, qv.w};
            float w4 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = ex2((l[e] - st.M) * st.s2) * st.invZ;
                w4 += fmaxf(p - qq[e], 0.f);
            }
            sum += (double)w4;
        }
        done = nv * 4;
    }
    for (int j = c0 + done + tid; j < c1; j += kBlock) sum += (double)wf(j);
    sum = wave_sum(sum);
    if (lane == 0) sm.wtot[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int w = 0; w < kWaves; ++w) tot += sm.wtot[w];
        a.resid[(size_t)b * kMaxSplits + s] = tot;
        __threadfence();
        const uint32_t t = atomicAdd(&a.ticketB[b], 1u);
        sm.last = t == (uint32_t)(S - 1);
    }
    __syncthreads();
    if (!sm.last) return;
    __threadfence();
    const double u = (double)a.coins[(size_t)b * R + G];
    if (tid == 0) {
        a.ticketB[b] = 0u;
        double tot = 0.0;
        for (int c = 0; c < S; ++c) tot += a.resid[(size_t)b * kMaxSplits + c];
        sm.fallback = !(tot > 0.0);
        if (!sm.fallback) {
            const double t = u * tot;
            double pre = 0.0, before = 0.0;
            int ss = -1, lastpos = -1;
            for (int c = 0; c < S; ++c) {
                const double Pc = a.resid[(size_t)b * kMaxSplits + c];
                if (Pc > 0.0) {
                    lastpos = c;
                    if (t <= pre + Pc) {
                        ss = c;
                        before = pre;
                        break;
                    }
                }
                pre += Pc;
            }
            if (ss < 0) {
                ss = lastpos;
                before = pre - a.resid[(size_t)b * kMaxSplits + ss];
            }
            sm.sstar = ss;
            sm.tau = t - before;
        }
    }
    __syncthreads();
    int y;
    if (sm.fallback) {  // residual mass not positive: draw from p_k itself
        const Part* pr = a.parts + ((size_t)b * R + k) * kMaxSplits;
        y = draw_row<T>(rowp, V, a.chunk, S, pr, st.M, st.s2, st.T, u, nullptr, 0, sm);
    } else {
        const int ss = sm.sstar;
        const int cs0 = ss * a.chunk, cs1 = min(V, cs0 + a.chunk);
        y = scan_find(wf, cs0, cs1, sm.tau, sm);
        if (y < 0) y = cs0;  // unreachable for a positive chunk mass
    }
    if (tid == 0) {
        a.out_tokens[(size_t)b * R + k] = y;
        if (a.probs) {
            const double l = (double)Ld<T>::one(rowp + y);
            a.probs[(size_t)b * R + k] = (float)(exp((l - (double)st.M) / st.T) / st.Z);
        }
    }
}

// ---------------------------------------------------------------------------------------
// k_tree: one workgroup per request

struct TreeSmem {
    int par[SPEC_MAX_N];
    int tok[SPEC_MAX_N];
    int anc[SPEC_MAX_N];
    int dep[SPEC_MAX_N];
    int kids[SPEC_MAX_N];
    int excl[SPEC_MAX_N];
    double pc[SPEC_MAX_N];
    int wcnt[kWaves];
    int chosen;
    int nkids;
    float M;
    double Z;
    int arg;
};

template <typename T>
__device__ void tree_row_stats(const KArgs& a, int b, int j, bool sampling, double Td, float s2,
                               TreeSmem& ts) {
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        const Part* pr = a.parts + ((size_t)b * a.R + j) * kMaxSplits;
        float m = -INFINITY;
        int ix = INT_MAX;
        double z = 0.0;
        if (lane < a.S) {
            m = pr[lane].m;
            ix = pr[lane].idx;
            z = pr[lane].z;
        }
        if (sampling) {
            const float M = wave_max(m);
            double term = 0.0;
            if (lane < a.S && m != -INFINITY) term = z * exp(((double)m - (double)M) / Td);
            const double Z = wave_sum(term);
            if (lane == 0) {
                ts.M = M;
                ts.Z = Z;
            }
        } else {
            wave_argmax(m, ix);
            if (lane == 0) {
                ts.M = m;
                ts.arg = ix;
            }
        }
    }
    (void)s2;
    __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_tree(KArgs a, int sampling) {
    __shared__ TreeSmem ts;
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const int N = a.R, V = a.V, D = a.D, S = a.S;
    const int32_t* par_g = a.parents + (size_t)b * N;
    const int32_t* tok_g = a.tokens + (size_t)b * N;
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
    bad = __syncthreads_or(bad);
    if (!bad) {  // depths by pointer jumping (parents[i] < i: every chain ends at the root)
        for (int i = tid; i < N; i += kBlock) {
            ts.anc[i] = i == 0 ? 0 : ts.par[i];
            ts.dep[i] = i == 0 ? 0 : 1;
        }
        for (int r = 1; r < N; r <<= 1) {
            __syncthreads();
            int nd[SPEC_MAX_N / kBlock], na[SPEC_MAX_N / kBlock];
            int c = 0;
            for (int i = tid; i < N; i += kBlock, ++c) {
                const int an = ts.anc[i];
                nd[c] = ts.dep[i] + (an == i ? 0 : ts.dep[an]);
                na[c] = ts.anc[an];
            }
            __syncthreads();
            c = 0;
            for (int i = tid; i < N; i += kBlock, ++c) {
                if (ts.anc[i] != i) {
                    ts.dep[i] = nd[c];
                    ts.anc[i] = na[c];
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < N; i += kBlock)
            if (ts.dep[i] > D) bad = true;
        // every row needs a finite logit
        for (int j = tid; j < N; j += kBlock) {
            const Part* pr = a.parts + ((size_t)b * N + j) * kMaxSplits;
            float m = -INFINITY;
            for (int s = 0; s < S; ++s) m = fmaxf(m, pr[s].m);
            if (m == -INFINITY) bad = true;
        }
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
        if (tid == 0) a.accept_len[b] = -1;
        return;
    }

    const T* logits = reinterpret_cast<const T*>(a.logits);
    const double Td = (double)Tf;
    const float s2 = kLog2e / Tf;
    int cur = 0, d = 0, nexcl = 0;
    for (;;) {
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
        tree_row_stats<T>(a, b, cur, sampling != 0, Td, s2, ts);
        const T* rowp = logits + ((size_t)b * N + cur) * V;
        if (sampling) {
            for (int j = tid; j < count; j += kBlock) {
                const double l = (double)Ld<T>::one(rowp + ts.tok[ts.kids[j]]);
                ts.pc[j] = exp((l - (double)ts.M) / Td) / ts.Z;
            }
            __syncthreads();
            if (tid == 0) {
                const double u = (double)a.coins[(size_t)b * (D + 1) + d];
                const double tha = (double)a.th_acc, ths = (double)a.th_single;
                double acc = 0.0;
                int ch = -1;
                for (int j = 0; j < count; ++j) {
                    acc += ts.pc[j];
                    if (u <= acc / tha || ts.pc[j] >= ths) {
                        ch = j;
                        break;
                    }
                }
                ts.chosen = ch;
            }
        } else if (tid == 0) {
            int ch = -1;
            for (int j = 0; j < count; ++j)
                if (ts.tok[ts.kids[j]] == ts.arg) {
                    ch = j;
                    break;
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
            if (probs) probs[d] = sampling ? (float)ts.pc[ch] : 0.f;
        }
        __syncthreads();
        cur = c;
        ++d;
    }

    // final token from row cur
    tree_row_stats<T>(a, b, cur, sampling != 0, Td, s2, ts);
    const T* rowp = logits + ((size_t)b * N + cur) * V;
    int y;
    float py = 0.f;
    if (sampling) {
        const Part* pr = a.parts + ((size_t)b * N + cur) * kMaxSplits;
        const double u = (double)a.coins[(size_t)b * (D + 1) + D];
        y = draw_row<T>(rowp, V, a.chunk, S, pr, ts.M, s2, Td, u, ts.excl, nexcl, sm);
        if (y >= 0) py = (float)(exp(((double)Ld<T>::one(rowp + y) - (double)ts.M) / Td) / ts.Z);
    } else {
        y = ts.arg;
    }
    if (tid == 0) {
        out[d] = y;
        if (probs) probs[d] = py;
        a.accept_len[b] = d;
    }
    for (int e = d + 1 + tid; e <= D; e += kBlock) {
        out[e] = -1;
        if (probs) probs[e] = 0.f;
    }
    for (int e = d + tid; e < D; e += kBlock) nodes[e] = -1;
}

__global__ void k_fill_zero(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------------------
// host side

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
    size_t ticketA, ticketB, parts, state, resid, total;
};

Layout layout_for(int B, int R) {
    Layout L;
    size_t off = 0;
    L.ticketA = off;
    off = align256(off + sizeof(uint32_t) * (size_t)B);
    L.ticketB = off;
    off = align256(off + sizeof(uint32_t) * (size_t)B);
    L.parts = off;
    off = align256(off + sizeof(Part) * (size_t)B * R * kMaxSplits);
    L.state = off;
    off = align256(off + sizeof(ResidState) * (size_t)B);
    L.resid = off;
    off = align256(off + sizeof(double) * (size_t)B * kMaxSplits);
    L.total = off;
    return L;
}

void bind_workspace(KArgs& a, void* ws, int B, int R) {
    const Layout L = layout_for(B, R);
    char* base = static_cast<char*>(ws);
    a.ticketA = reinterpret_cast<uint32_t*>(base + L.ticketA);
    a.ticketB = reinterpret_cast<uint32_t*>(base + L.ticketB);
    a.parts = reinterpret_cast<Part*>(base + L.parts);
    a.state = reinterpret_cast<ResidState*>(base + L.state);
    a.resid = reinterpret_cast<double*>(base + L.resid);
}

// Split each row into S chunks of `chunk` elements (a multiple of 8): about 32 KB of
// logits per workgroup, at least ~2048 workgroups in flight, and at least 1024
// elements per chunk.  SPEC_VERIFY_SPLITS overrides the count (launch-shape sweeps).
void choose_split(long rows, int V, int esize, int* S_out, int* chunk_out) {
    const long row_bytes = (long)V * esize;
    long s = (row_bytes + 32 * 1024 - 1) / (32 * 1024);
    const long min_wgs = 2048;
    if (rows * s < min_wgs) s = (min_wgs + rows - 1) / rows;
    const long by_size = V / 1024 > 1 ? V / 1024 : 1;
    if (s > by_size) s = by_size;
    if (const char* env = std::getenv("SPEC_VERIFY_SPLITS")) {
        const long e = std::atol(env);
        if (e >= 1) s = e;
    }
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < 1) s = 1;
    long ch = ((long)V + s - 1) / s;
    ch = (ch + 7) / 8 * 8;
    s = ((long)V + ch - 1) / ch;
    *S_out = (int)s;
    *chunk_out = (int)ch;
}

int check_common(const void* logits, int dtype, int B, int V, void* ws, size_t ws_bytes,
                 int op, int R) {
    if (!logits || (B > 0 && !ws)) return SPEC_ERR_NULL;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
    if (B < 0 || V < 1) return SPEC_ERR_SHAPE;
    const size_t es = dtype == SPEC_F32 ? 4 : 2;
    if (((uintptr_t)logits) % es) return SPEC_ERR_PARAM;
    if ((long long)B * R * kMaxSplits > (long long)INT_MAX) return SPEC_ERR_SHAPE;
    if (B > 0) {
        if (((uintptr_t)ws) % 256) return SPEC_ERR_WORKSPACE;
        if (ws_bytes < spec_workspace_bytes(op, B, R, V)) return SPEC_ERR_WORKSPACE;
    }
    return SPEC_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP; }

template <typename T>
int run_greedy(KArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_rows<T, kGreedyChain>), dim3(a.B * a.R * a.S), dim3(kBlock), 0, st, a);
    return launch_status();
}

template <typename T>
int run_chain(KArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_rows<T, kSamplingChain>), dim3(a.B * a.R * a.S), dim3(kBlock), 0, st, a);
    int rc = launch_status();
    if (rc != SPEC_OK) return rc;
    hipLaunchKernelGGL((k_residual<T>), dim3(a.B * a.S), dim3(kBlock), 0, st, a);
    return launch_status();
}

template <typename T>
int run_tree(KArgs& a, int sampling, hipStream_t st) {
    if (sampling)
        hipLaunchKernelGGL((k_rows<T, kRowsOnlySampling>), dim3(a.B * a.R * a.S), dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL((k_rows<T, kRowsOnlyGreedy>), dim3(a.B * a.R * a.S), dim3(kBlock), 0, st, a);
    int rc = launch_status();
    if (rc != SPEC_OK) return rc;
    hipLaunchKernelGGL((k_tree<T>), dim3(a.B), dim3(kBlock), 0, st, a, sampling);
    return launch_status();
}

}  // namespace

// ---------------------------------------------------------------------------------------
// C ABI

extern "C" size_t spec_workspace_bytes(int op, int B, int R, int V) {
    if (B < 0 || R < 1 || V < 1) return 0;
    if (op == SPEC_OP_GREEDY || op == SPEC_OP_CHAIN) {
        if (R - 1 < 1 || R - 1 > SPEC_MAX_G) return 0;
    } else if (op == SPEC_OP_TREE) {
        if (R > SPEC_MAX_N) return 0;
    } else {
        return 0;
    }
    return layout_for(B, R).total;
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
        default: return "unknown status";
    }
}

extern "C" int spec_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
    if (!workspace) return SPEC_ERR_NULL;
    if (((uintptr_t)workspace) % 4) return SPEC_ERR_PARAM;
    const size_t n = ws_bytes / 4;
    if (n == 0) return SPEC_OK;
    size_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint32_t*>(workspace), n);
    return launch_status();
}

extern "C" int spec_verify_greedy(const void* logits, int dtype, const int32_t* draft_tokens,
                                  int B, int G, int V, int32_t* accept_len, int32_t* out_tokens,
                                  void* workspace, size_t ws_bytes, void* stream) {
    if (!draft_tokens || !accept_len || !out_tokens) return SPEC_ERR_NULL;
    if (G < 1 || G > SPEC_MAX_G) return SPEC_ERR_SHAPE;
    int rc = check_common(logits, dtype, B, V, workspace, ws_bytes, SPEC_OP_GREEDY, G + 1);
    if (rc != SPEC_OK || B == 0) return rc;
    KArgs a = {};
    a.logits = logits;
    a.tokens = draft_tokens;
    a.B = B;
    a.R = G + 1;
    a.V = V;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    choose_split((long)B * a.R, V, dtype == SPEC_F32 ? 4 : 2, &a.S, &a.chunk);
    bind_workspace(a, workspace, B, a.R);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return dtype == SPEC_F32 ? run_greedy<float>(a, st) : run_greedy<uint16_t>(a, st);
}

extern "C" int spec_verify_chain(const void* logits, int dtype, const float* draft_probs,
                                 const int32_t* draft_tokens, const float* coins,
                                 const float* temperature, int B, int G, int V,
                                 int32_t* accept_len, int32_t* out_tokens, float* probs_out,
                                 void* workspace, size_t ws_bytes, void* stream) {
    if (!draft_probs || !draft_tokens || !coins || !temperature || !accept_len || !out_tokens)
        return SPEC_ERR_NULL;
    if (G < 1 || G > SPEC_MAX_G) return SPEC_ERR_SHAPE;
    int rc = check_common(logits, dtype, B, V, workspace, ws_bytes, SPEC_OP_CHAIN, G + 1);
    if (rc != SPEC_OK || B == 0) return rc;
    if (((uintptr_t)draft_probs) % 4) return SPEC_ERR_PARAM;
    KArgs a = {};
    a.logits = logits;
    a.q = draft_probs;
    a.tokens = draft_tokens;
    a.coins = coins;
    a.temperature = temperature;
    a.B = B;
    a.R = G + 1;
    a.V = V;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.probs = probs_out;
    choose_split((long)B * a.R, V, dtype == SPEC_F32 ? 4 : 2, &a.S, &a.chunk);
    bind_workspace(a, workspace, B, a.R);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return dtype == SPEC_F32 ? run_chain<float>(a, st) : run_chain<uint16_t>(a, st);
}

extern "C" int spec_verify_tree(const void* logits, int dtype, const int32_t* node_tokens,
                                const int32_t* parents, const float* coins,
                                const float* temperature, int B, int N, int V, int D, int mode,
                                float threshold_single, float threshold_acc,
                                int32_t* accept_len, int32_t* out_tokens,
                                int32_t* accepted_nodes, float* probs_out, void* workspace,
                                size_t ws_bytes, void* stream) {
    if (!node_tokens || !parents || !accept_len || !out_tokens || !accepted_nodes)
        return SPEC_ERR_NULL;
    if (mode != SPEC_TREE_GREEDY && mode != SPEC_TREE_SAMPLING) return SPEC_ERR_PARAM;
    if (mode == SPEC_TREE_SAMPLING) {
        if (!coins || !temperature) return SPEC_ERR_NULL;
        if (!(threshold_single > 0.f) || !(threshold_acc > 0.f)) return SPEC_ERR_PARAM;
    }
    if (N < 1 || N > SPEC_MAX_N || D < 1 || D > SPEC_MAX_N) return SPEC_ERR_SHAPE;
    int rc = check_common(logits, dtype, B, V, workspace, ws_bytes, SPEC_OP_TREE, N);
    if (rc != SPEC_OK || B == 0) return rc;
    KArgs a = {};
    a.logits = logits;
    a.tokens = node_tokens;
    a.parents = parents;
    a.coins = coins;
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
    choose_split((long)B * N, V, dtype == SPEC_F32 ? 4 : 2, &a.S, &a.chunk);
    bind_workspace(a, workspace, B, N);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return dtype == SPEC_F32 ? run_tree<float>(a, mode, st) : run_tree<uint16_t>(a, mode, st);
}
