// libi4decode: kernels and the C ABI of include/i4decode.h (gfx950).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <math.h>
#include <cmath>

#include <algorithm>
#include <mutex>
#include <vector>
#include <string.h>

#include "../../include/i4decode.h"
#include "attention.h"
#include "common.h"
#include "gemv.h"
#include "mfma.h"
#include "prefill.h"
#include "stream.h"

namespace {

#ifndef I4D_GEMV_NT
#define I4D_GEMV_NT 512
#endif
#ifndef I4D_GEMV_D
#define I4D_GEMV_D 6
#endif
#ifndef I4D_ATTN_NT
#define I4D_ATTN_NT 512
#endif
#ifndef I4D_WG_PER_CU
#define I4D_WG_PER_CU 1
#endif
constexpr int GEMV_NT = I4D_GEMV_NT;       // threads per GEMV workgroup
constexpr int GEMV_D = I4D_GEMV_D;         // units in flight per lane
constexpr int ATTN_NT = I4D_ATTN_NT;       // threads per attention workgroup
// the attention merge gives each (query head, 4 dims) slot its own thread:
// G <= 16 query heads per KV head at head_dim 128
static_assert(ATTN_NT >= 16 * 128 / 4, "attention workgroup smaller than its merge");
constexpr int WG_PER_CU = I4D_WG_PER_CU;   // GEMV workgroups per compute unit
constexpr int NSPLIT_MAX = 128;    // key-axis splits per (sequence, KV head)
constexpr int MAX_BATCH = 8;          // matrix-vector (VALU) path
constexpr int MAX_BATCH_ALL = 32;     // batches above MAX_BATCH take the MFMA path

template <int NB> struct MaxJ { static constexpr int v = NB <= 2 ? 8 : 4; };

// LDS beyond the staged activations: per-slot partials, a reduction scratch
// and an "extra" area (positions: 64 B; RoPE cos/sin table: NB * 64 float2).
constexpr int GEMV_EXTRA = 64 + MAX_BATCH * 64 * 8;


// ============================================================== epilogues and staging functors

// Stage `src` (optionally RMS-normalised with `gain`) into LDS.
template <int FMT, int NB, int PREC, int PC = PRE_CHUNKS>
struct StageFn {
    typedef StagePre<FMT, PC> Pre;
    char* act; const float* src; int stride; int K; int nb; const uint16_t* gain; float eps; float* red;
    I4D_DEVINL void issue(Pre& pre) { stage_issue<FMT, NB, GEMV_NT, PC>(pre, src, stride, K, nb, gain); }
    I4D_DEVINL void finish(const Pre& pre) {
        stage_finish<FMT, NB, GEMV_NT, PREC, PC>(pre, act, src, stride, K, nb, gain, eps, red);
    }
};

// Activation precision of the int4 dot products: one fp16 plane (about 2^-12
// relative per input), or fp16 value + fp16 remainder (about 2^-22) for the
// q/k/v projection, whose k and v are rounded to bf16 into the cache.
constexpr int PREC_STD = 1, PREC_QKV = 2;

// y[b][row] = (resid ? resid[b][row] : 0) + W x   for rows 2p, 2p+1
// WT: outputs are read by other workgroups of the same launch (persistent
// kernel) and are written through; one launch per phase stores plainly.
template <bool WT = true>
struct EpiRows {
    float* y; const float* resid; int n; int nb;
    I4D_DEVINL void operator()(int, int pair, int b, float va, float vb) {
        if (b >= nb) return;
        const int r = 2 * pair;
        float* yr = y + (size_t)b * n;
        const float* rr = resid ? resid + (size_t)b * n : nullptr;
        st_out<WT>(yr + r, (rr ? rr[r] : 0.f) + va);
        if (r + 1 < n) st_out<WT>(yr + r + 1, (rr ? rr[r + 1] : 0.f) + vb);
    }
    I4D_DEVINL void end_pass(int, int, int) {}
};

// act[b][i] = SiLU(gate_i) * up_i
template <bool WT = true>
struct EpiSwiGLU {
    float* act; int F; int nb;
    I4D_DEVINL void operator()(int, int pair, int b, float g, float u) {
        if (b >= nb) return;
        st_out<WT>(act + (size_t)b * F + pair, g / (1.0f + expf(-g)) * u);
    }
    I4D_DEVINL void end_pass(int, int, int) {}
};

// cos/sin of the RoPE angles pos[b] * base^(-2i/hd) for every batch slot and
// pair index i < hd/2, computed once per launch in float64 (the angle reaches
// 3e4 rad at long positions, beyond what float32 can reduce accurately) and
// kept in LDS as float2 [NB][hd/2].  pos_lds[b] = -1 (invalid) uses angle 0.
template <int NB>
I4D_DEVINL void rope_table(float2* cs, const int* pos_lds, int hd, double base) {
    const int half = hd >> 1;
    for (int idx = i4d_tid(); idx < NB * half; idx += blockDim.x) {
        const int b = idx / half, i = idx - b * half;
        const double theta = pow(base, -2.0 * (double)i / (double)hd);
        const double phi = (double)max(pos_lds[b], 0) * theta;
        double sn, cn;
        sincos(phi, &sn, &cn);             // one argument reduction for both
        cs[idx] = float2{(float)cn, (float)sn};
    }
}

// Positions of the batch into LDS (an invalid one becomes -1 and raises the
// status word), then the cos/sin table for them.
template <int NB>
struct RopeSetup {
    const int* pos; int* pos_lds; float2* cs; int* status; int nb, max_pos, cap, hd; double base;
    I4D_DEVINL void operator()() const {
        if (i4d_tid() < NB) {
            int p = -1;
            if (i4d_tid() < nb) {
                p = pos[i4d_tid()];
                if (p < 0 || p > max_pos || p >= cap) {
                    if (blockIdx.x == 0) raise_status(status, I4D_DEV_BAD_POS);
                    p = -1;
                }
            }
            pos_lds[i4d_tid()] = p;
        }
        __syncthreads();
        rope_table<NB>(cs, pos_lds, hd, base);
    }
};

// RoPE on q and k pairs, q to the fp32 buffer, bf16 k/v appended at slot pos[b].
template <bool WT = true>
struct EpiQKV {
    float* q; uint16_t* kc; uint16_t* vc; uint16_t* kvn; const int* pos_lds; const float2* cs;
    int cap, hq, hkv, hd, nb;
    int kvb;                   // 1: sequence b appends to cache b; 0: all append to cache 0 (a prompt chunk)
    KvMap pg;                  // paged cache (pg.pages == nullptr: contiguous)
    int* status;               // I4D_DEV_BAD_PAGE when a page id is out of range (the append is dropped)
    I4D_DEVINL void operator()(int, int pair, int b, float va, float vb) {
        if (b >= nb) return;
        const int half = hd >> 1;
        const int npq = hq * half, npk = hkv * half;
        int lp = pair, mat = 0;
        if (lp >= npq) { lp -= npq; mat = 1; if (lp >= npk) { lp -= npk; mat = 2; } }
        const int head = lp / half, i = lp - head * half;
        const int p = pos_lds[b];                      // -1: invalid position, nothing appended
        float ra = va, rb = vb;
        if (mat < 2) {
            const float2 r = cs[b * half + i];
            ra = va * r.x - vb * r.y;
            rb = va * r.y + vb * r.x;
        }
        if (mat == 0) {
            float* qr = q + ((size_t)b * hq + head) * hd;
            st_out<WT>(qr + i, ra); st_out<WT>(qr + i + half, rb);
        } else if (p >= 0) {
            const uint16_t ba = f32_to_bf16(ra), bb = f32_to_bf16(rb);
            if (kvn != nullptr) {                      // side copy for this step's attention (none for a prompt)
                uint16_t* nr = kvn + (((size_t)b * hkv + head) * 2 + (mat - 1)) * hd;
                st_out<WT>(nr + i, ba); st_out<WT>(nr + i + half, bb);
            }
            // 16-position tiles: K [hd/32][16][32], V [hd][16]
            bool bad = false;
            const size_t tile = kv_tile_off(pg, cap, hkv, hd, b * kvb, head, p >> 4, bad);
            if (bad) {
                if (status && i == 0) raise_status(status, I4D_DEV_BAD_PAGE);
                return;
            }
            const int tp = p & 15;
            if (mat == 1) {
                uint16_t* kt = kc + tile;
                st_out<WT>(kt + (i >> 5) * 512 + tp * 32 + (i & 31), ba);
                st_out<WT>(kt + ((i + half) >> 5) * 512 + tp * 32 + ((i + half) & 31), bb);
            } else {
                uint16_t* vt = vc + tile;
                st_out<WT>(vt + (size_t)i * 16 + tp, ba);
                st_out<WT>(vt + (size_t)(i + half) * 16 + tp, bb);
            }
        }
    }
    I4D_DEVINL void end_pass(int, int, int) {}
};

// greedy argmax over rows 2p, 2p+1: per-thread running best key of batch slot
// `bslot` (a thread always serves the same slot: the epilogue's thread-to-slot
// assignment repeats every pass)
struct EpiArgmax {
    int n; int nb; u64 best; int bslot; Sampler smp;
    I4D_DEVINL void operator()(int, int pair, int b, float va, float vb) {
        if (b >= nb) return;
        const int r = 2 * pair;
        u64 k = argmax_key(smp.score(va, b, (u32)r), (u32)r);
        if (r + 1 < n) { const u64 k2 = argmax_key(smp.score(vb, b, (u32)(r + 1)), (u32)(r + 1)); k = k2 > k ? k2 : k; }
        best = k > best ? k : best;
        bslot = b;
    }
    I4D_DEVINL void end_pass(int, int, int) {}
};

// ============================================================== LDS carve-up for GEMV kernels
template <int FMT, int NB, int NT = GEMV_NT>
__host__ __device__ constexpr int gemv_part_bytes() { return (NT / 16) * (MaxJ<NB>::v * NB * 2 + 2) * 4; }

template <int FMT, int NB, int PREC>
__host__ inline size_t gemv_lds_bytes(int K) {
    return (size_t)act_lds_bytes<FMT, NB, PREC>(K) + gemv_part_bytes<FMT, NB>() + (GEMV_NT / 64) * NB * 4 + GEMV_EXTRA;
}

struct GemvLds { char* act; float* part; float* red; char* extra; };

template <int FMT, int NB, int PREC>
I4D_DEVINL GemvLds carve(char* lds, int K) {
    GemvLds l;
    l.act = lds;
    l.part = (float*)(lds + act_lds_bytes<FMT, NB, PREC>(K));
    l.red = l.part + gemv_part_bytes<FMT, NB>() / 4;
    l.extra = (char*)(l.red + (GEMV_NT / 64) * NB);
    return l;
}

// ============================================================== kernels
__global__ void k_fill_zero(int* p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + i4d_tid(); i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void k_dequant(const uint8_t* codes, const uint16_t* scales, int n, int k, int group, int ngroups, float* out) {
    const size_t total = (size_t)n * k;
    for (size_t idx = blockIdx.x * (size_t)blockDim.x + i4d_tid(); idx < total; idx += (size_t)gridDim.x * blockDim.x) {
        const size_t r = idx / k;
        const int i = (int)(idx - r * k);
        const uint8_t byte = codes[r * (size_t)(k >> 1) + (i >> 1)];
        const int c = (i & 1) ? (byte >> 4) : (byte & 15);
        out[idx] = (float)(c - 8) * bf16_to_f32(scales[r * ngroups + i / group]);
    }
}

template <int FMT, int NB>
__global__ void __launch_bounds__(GEMV_NT) k_gemv_rows(GemvTask t, const float* x, int x_stride, int nb,
                                                        const uint16_t* gain, float eps, float* y, const float* resid) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    GemvLds L = carve<FMT, NB, PREC_STD>(lds, t.k);
    StageFn<FMT, NB, PREC_STD> st{L.act, x, x_stride, t.k, nb, gain, eps, L.red};
    EpiRows<false> ep{y, resid, t.a.n, nb};
    gemv_run<FMT, NB, PREC_STD, GEMV_NT, GEMV_D, MaxJ<NB>::v, KIND_ADJ>(t, blockIdx.x, gridDim.x, L.act, L.part, st, ep);
}

template <int FMT, int NB>
__global__ void __launch_bounds__(GEMV_NT) k_gemv_swiglu(GemvTask t, const float* x, int nb, const uint16_t* gain, float eps, float* act) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    GemvLds L = carve<FMT, NB, PREC_STD>(lds, t.k);
    StageFn<FMT, NB, PREC_STD> st{L.act, x, t.k, t.k, nb, gain, eps, L.red};
    EpiSwiGLU<false> ep{act, t.a.n, nb};
    gemv_run<FMT, NB, PREC_STD, GEMV_NT, GEMV_D, MaxJ<NB>::v, KIND_TWO>(t, blockIdx.x, gridDim.x, L.act, L.part, st, ep);
}

template <int FMT, int NB>
__global__ void __launch_bounds__(GEMV_NT) k_gemv_qkv(GemvTask t, const float* x, int nb, const uint16_t* gain, float eps,
                                                       const int* pos, int max_pos, float* q, uint16_t* kc, uint16_t* vc,
                                                       uint16_t* kvn, int cap, int hq, int hkv, double base, int* status, int kvb,
                                                       KvMap pgm) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    GemvLds L = carve<FMT, NB, PREC_QKV>(lds, t.k);
    int* pos_lds = (int*)L.extra;
    float2* cs = (float2*)(L.extra + 64);
    RopeSetup<NB>{pos, pos_lds, cs, status, nb, max_pos, cap, t.head_dim, base}();
    StageFn<FMT, NB, PREC_QKV> st{L.act, x, t.k, t.k, nb, gain, eps, L.red};
    EpiQKV<false> ep{q, kc, vc, kvn, pos_lds, cs, cap, hq, hkv, t.head_dim, nb, kvb, pgm, status};
    gemv_run<FMT, NB, PREC_QKV, GEMV_NT, GEMV_D, MaxJ<NB>::v, KIND_QKV>(t, blockIdx.x, gridDim.x, L.act, L.part, st, ep);
}

template <int FMT, int NB>
__global__ void __launch_bounds__(GEMV_NT) k_lm_head(GemvTask t, const float* h, int nb, u64* wg_keys, Sampler smp) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    GemvLds L = carve<FMT, NB, PREC_STD>(lds, t.k);
    StageFn<FMT, NB, PREC_STD> st{L.act, h, t.k, t.k, nb, nullptr, 0.f, L.red};
    EpiArgmax ep{t.a.n, nb, 0ull, -1, smp};
    gemv_run<FMT, NB, PREC_STD, GEMV_NT, GEMV_D, MaxJ<NB>::v, KIND_ADJ>(t, blockIdx.x, gridDim.x, L.act, L.part, st, ep);
    // workgroup best per batch slot -> this workgroup's key slots
    u64* kl = (u64*)(L.extra + GEMV_EXTRA);
    int* ks = (int*)(kl + GEMV_NT);
    kl[i4d_tid()] = ep.best;
    ks[i4d_tid()] = ep.bslot;
    __syncthreads();
    if (i4d_tid() < MAX_BATCH) {
        u64 best = 0;
        for (int i = 0; i < GEMV_NT; ++i)
            if (ks[i] == i4d_tid()) best = kl[i] > best ? kl[i] : best;
        wg_keys[(size_t)blockIdx.x * MAX_BATCH + i4d_tid()] = best;
    }
}

// Reduce the per-workgroup argmax keys: token = lowest id of the largest logit.
__global__ void __launch_bounds__(256) k_lm_finalize(const u64* wg_keys, int nwg, int kstride, int nb, int32_t* token_out, float* max_out) {
    __shared__ u64 red[256];
    for (int b = 0; b < nb; ++b) {
        u64 best = 0;
        for (int w = i4d_tid(); w < nwg; w += 256) {
            const u64 k = wg_keys[(size_t)w * kstride + b];
            best = k > best ? k : best;
        }
        red[i4d_tid()] = best;
        __syncthreads();
        for (int s2 = 128; s2 > 0; s2 >>= 1) {
            if (i4d_tid() < s2) red[i4d_tid()] = red[i4d_tid() + s2] > red[i4d_tid()] ? red[i4d_tid() + s2] : red[i4d_tid()];
            __syncthreads();
        }
        if (i4d_tid() == 0) {
            const u64 k = red[0];
            token_out[b] = (int32_t)(0xFFFFFFFFu - (u32)(k & 0xFFFFFFFFull));
            max_out[b] = float_from_order_key((u32)(k >> 32));
        }
        __syncthreads();
    }
}

template <int HD, bool PAGED>
__global__ void __launch_bounds__(ATTN_NT) k_attention(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int NSW = AttnNsw<ATTN_NT>::v;
    const int items = a.batch * a.hkv * a.nsplit;
    AttnRegs<HD, NSW> R;
    for (int it = blockIdx.x; it < items; it += gridDim.x) attn_item<HD, ATTN_NT, NSW, PAGED>(a, it, lds, R, false);
}

// ---------------------------------------------------------------- streaming-read probe
// Each lane keeps four 16-byte nontemporal loads in flight over a grid-stride
// sweep; the words are XOR-folded so the loads cannot be dropped.
__global__ void __launch_bounds__(512) k_read_probe(const u32x4* src, size_t n16, u32* sink) {
    const size_t nthr = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + i4d_tid();
    u32 acc = 0;
    for (; i + 3 * nthr < n16; i += 4 * nthr) {
        const u32x4 a = ld_g_nt(src + i), b = ld_g_nt(src + i + nthr), c = ld_g_nt(src + i + 2 * nthr),
                    d = ld_g_nt(src + i + 3 * nthr);
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += nthr) {
        const u32x4 a = ld_g_nt(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int m = 32; m >= 1; m >>= 1) acc ^= (u32)__shfl_xor((int)acc, m, 64);
    if ((i4d_tid() & 63) == 0) atomicXor(sink, acc);
}

// ---------------------------------------------------------------- decode loop glue
// x[b] = row tokens[b] of the bf16 embedding table (an id outside the table
// gives a zero row and the status bit).
__global__ void __launch_bounds__(256) k_embed(const uint16_t* table, int vocab, int D, const int* tokens, float* x, int* status) {
    const int b = blockIdx.y;
    const int t = tokens[b];
    const bool ok = t >= 0 && t < vocab;
    if (!ok && blockIdx.x == 0 && i4d_tid() == 0) raise_status(status, I4D_DEV_BAD_TOKEN);
    const uint16_t* row = table + (size_t)(ok ? t : 0) * D;
    for (int d = blockIdx.x * 256 + i4d_tid(); d < D; d += gridDim.x * 256) x[(size_t)b * D + d] = ok ? bf16_to_f32(row[d]) : 0.f;
}

// every sequence moves on to its next position
__global__ void __launch_bounds__(64) k_advance(int* pos, int nb) {
    if (i4d_tid() < nb) pos[i4d_tid()] += 1;
}

// ---------------------------------------------------------------- top-k sampling
// Top-k sampling (the decode loop's sample step restricted to the k largest
// logits, renormalised): the logits of a step are written by the LM head's
// GEMV, every 1024-row slice keeps its k largest ordered keys (logit, then
// lower id: argmax_key), one workgroup per sequence merges the slices' lists
// into the global k largest, and the token is the Gumbel-max over those k
// rows (the noise of Sampler::score, so k = V gives the temperature draw and
// k = 1 the greedy token).
constexpr int TOPK_MAX = 64, TOPK_SLICE = 1024, TOPK_MERGE_MAX = 16384;

// Bitonic sort of n (a power of two) keys in LDS into descending order.
I4D_DEVINL void bitonic_desc(u64* key, int n) {
    for (int size = 2; size <= n; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < (n >> 1); t += blockDim.x) {
                const int i = 2 * t - (t & (stride - 1)), j = i + stride;
                const bool desc = (i & size) == 0;
                const u64 a = key[i], c = key[j];
                if ((a < c) == desc) { key[i] = c; key[j] = a; }
            }
            __syncthreads();
        }
}

// grid (slices, B): the k largest keys of rows [1024 s, 1024 s + 1024) of
// sequence b's logits into cand[b][s][0..k) (key 0 pads past the vocabulary)
__global__ void __launch_bounds__(512) k_topk_slice(const float* logits, int V, int k, u64* cand) {
    __shared__ u64 key[TOPK_SLICE];
    const int sl = blockIdx.x, b = blockIdx.y, nsl = gridDim.x;
    for (int i = threadIdx.x; i < TOPK_SLICE; i += blockDim.x) {
        const int row = sl * TOPK_SLICE + i;
        key[i] = row < V ? argmax_key(ld_g(logits + (size_t)b * V + row), (u32)row) : 0ull;
    }
    __syncthreads();
    bitonic_desc(key, TOPK_SLICE);
    for (int i = threadIdx.x; i < k; i += blockDim.x) cand[((size_t)b * nsl + sl) * k + i] = key[i];
}

// grid (B): merge sequence b's n = slices * k candidate keys (n padded to the
// power of two np2 in LDS), keep the k largest, and draw among them
__global__ void __launch_bounds__(1024) k_topk_sample(const u64* cand, int n, int np2, int k, Sampler smp, int32_t* token_out,
                                                      float* score_out) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    u64* key = (u64*)lds;
    __shared__ u64 wbest[16];
    const int b = blockIdx.x, tid = threadIdx.x;
    for (int i = tid; i < np2; i += blockDim.x) key[i] = i < n ? ld_g(cand + (size_t)b * n + i) : 0ull;
    __syncthreads();
    bitonic_desc(key, np2);
    u64 best = 0;
    if (tid < k && key[tid] != 0ull) {
        const u64 kk = key[tid];
        const u32 row = 0xFFFFFFFFu - (u32)kk;
        const float logit = float_from_order_key((u32)(kk >> 32));
        best = argmax_key(smp.score(logit, b, row), row);
    }
    for (int o = 32; o >= 1; o >>= 1) {
        const u32 lo = __shfl_xor((u32)best, o, 64), hi = __shfl_xor((u32)(best >> 32), o, 64);
        const u64 other = ((u64)hi << 32) | lo;
        best = other > best ? other : best;
    }
    if ((tid & 63) == 0) wbest[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        u64 m = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = wbest[w] > m ? wbest[w] : m;
        token_out[b] = (int32_t)(0xFFFFFFFFu - (u32)m);
        score_out[b] = float_from_order_key((u32)(m >> 32));
    }
}

// ---------------------------------------------------------------- batched (MFMA) phases
template <int NB>
__global__ void __launch_bounds__(512) k_mfma_rows(MfmaTask m, float* y, const float* resid) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    EpiRows<false> ep{y, resid, m.t.a.n, m.nb};
    mfma_gemm<KIND_ADJ, NB, 1, MEPI_FN>(m, lds, ep, nullptr);
}

template <int NB>
__global__ void __launch_bounds__(512) k_mfma_swiglu(MfmaTask m, float* act) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    EpiSwiGLU<false> ep{act, m.t.a.n, m.nb};
    mfma_gemm<KIND_TWO, NB, 1, MEPI_FN>(m, lds, ep, nullptr);
}

// q/k/v with RoPE and the KV append; positions (validated, -1 = skipped) and
// the cos/sin table come from the staging kernel
template <int NB>
__global__ void __launch_bounds__(512) k_mfma_qkv(MfmaTask m, float* q, uint16_t* kc, uint16_t* vc, uint16_t* kvn,
                                                  const int* posv, const float2* cs, int cap, int hq, int hkv, int kvb,
                                                  KvMap pgm, int* status) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    EpiQKV<false> ep{q, kc, vc, kvn, posv, cs, cap, hq, hkv, m.t.head_dim, m.nb, kvb, pgm, status};
    mfma_gemm<KIND_QKV, NB, 2, MEPI_FN>(m, lds, ep, nullptr);
}

template <int NB>
__global__ void __launch_bounds__(512) k_mfma_lm(MfmaTask m, u64* wg_keys, Sampler smp) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    mfma_gemm<KIND_ADJ, NB, 1, MEPI_ARGMAX>(m, lds, smp, wg_keys);
}

// Workspace: a 16 KB header (status word, the streaming kernel's launch epoch,
// the attention arrival counters, the batched GEMM's row-block counters),
// then one region of buffers per layer, then (batch 1) the streaming kernel's
// region.  The LM head uses the bytes after the header for its per-workgroup
// argmax keys (WS_LM_BYTES), overlapping the layer buffers: calls on one
// stream never use both at once.  The counters sit in the header because
// they must read zero at the start of every attention phase (each merge
// resets its own).
constexpr size_t WS_STATUS = 0, WS_EPOCH = 64, WS_CNT = 1024, WS_CNT_END = 4096, WS_MCNT = 8192, WS_HEADER = 16384;
constexpr int WS_MAX_CNT = (int)((WS_CNT_END - WS_CNT) / 4);   // B * Hkv arrival counters
constexpr int WS_MAX_MCNT = (int)((WS_HEADER - WS_MCNT) / 4);  // row-block arrival counters of the batched GEMM
constexpr int LM_MAX_WG = 4096;
constexpr size_t WS_LM_KEYS = WS_HEADER, WS_LM_BYTES = (size_t)LM_MAX_WG * MAX_BATCH_ALL * 8;
constexpr size_t WS_LM_END = WS_LM_KEYS + WS_LM_BYTES;   // batched-GEMM scratch of the LM head and the GEMV hook

// ============================================================== host helpers
int g_num_cus[64];

int num_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (g_num_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_num_cus[dev] = n;
    }
    return g_num_cus[dev];
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t stream;                        // the streaming kernel's region (batch 1), 0 if none
    size_t mfma;                          // scratch of the batched (MFMA) phases, batches above MAX_BATCH
    size_t layer0, layer_stride;          // per-layer regions
    size_t q, o, y, act, x, kvn, pm, pl, po;   // offsets inside a layer region
    int pstride;                          // attention partials per head (>= splits, multiple of 32)
    size_t total;
};

int nb_mfma(int batch);
size_t layer_scratch_bytes(const i4d_config* c, int nb);

// Most key-axis splits plan_attention picks for this shape and batch.
int attn_splits_max(const i4d_config* c, int B) {
    const int want = (num_cus() + B * c->n_kv_heads - 1) / (B * c->n_kv_heads);
    return std::max(1, std::min(want, NSPLIT_MAX));
}

// Layer l's region holds its q, merged attention output o, residual y, SwiGLU
// activations, output x, the new token's k/v side copy and the attention
// partials.  Partial rows are padded to 128-byte lines so the partials of
// different (sequence, KV head) groups never share a cache line.  The
// streaming kernel's region comes after everything the LM head may overlay.
WsLayout ws_layout(const i4d_config* c, int n_layers, int B) {
    WsLayout w;
    size_t off = WS_HEADER;
    const size_t hq = c->n_q_heads, hkv = c->n_kv_heads, hd = c->head_dim;
    w.pstride = (attn_splits_max(c, B) + 31) / 32 * 32;
    size_t lo = 0;
    auto ltake = [&](size_t bytes) { size_t o = lo; lo = align256(lo + bytes); return o; };
    w.q = ltake((size_t)B * hq * hd * 4);
    w.o = ltake((size_t)B * hq * hd * 4);
    w.y = ltake((size_t)B * c->d_model * 4);
    w.act = ltake((size_t)B * c->d_ff * 4);
    w.x = ltake((size_t)B * c->d_model * 4);
    w.kvn = ltake((size_t)B * hkv * 2 * hd * 2);
    w.pm = ltake((size_t)B * hq * w.pstride * 4);
    w.pl = ltake((size_t)B * hq * w.pstride * 4);
    w.po = ltake((size_t)B * hq * w.pstride * hd * 4);
    w.layer_stride = lo;
    w.layer0 = off;
    off += (size_t)std::max(n_layers, 1) * lo;
    w.mfma = 0;
    if (B > MAX_BATCH / 2) {              // after the LM head's keys, which overlay the layer regions
        off = std::max(off, WS_LM_END);
        w.mfma = off;
        off += layer_scratch_bytes(c, nb_mfma(B));
    }
    off = std::max(off, WS_LM_END);
    w.stream = 0;
    if (B == 1 && c->head_dim == 128) {
        w.stream = align256(off);
        off = w.stream + i4d_stream::region_bytes(c, std::max(n_layers, 1), num_cus());
    }
    w.total = off;
    return w;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int v) { int l = 0; while ((1 << l) < v) ++l; return l; }

int validate_mat(const i4d_mat* m, int n, int k, int dtype, int group) {
    if (!m || !m->data) return I4D_EINVAL;
    if (m->n != n || m->k != k || m->dtype != dtype) return I4D_EINVAL;
    if (!aligned(m->data, 16)) return I4D_EALIGN;
    if (dtype == I4D_WEIGHT_INT4) {
        if (!m->scales || m->group != group || group <= 0 || group % 8 != 0 || k % 8 != 0) return I4D_EINVAL;
        if (!aligned(m->scales, 2)) return I4D_EALIGN;
    } else if (dtype == I4D_WEIGHT_BF16) {
        if (k % 8 != 0) return I4D_EINVAL;
    } else {
        return I4D_EINVAL;
    }
    return I4D_OK;
}

int validate_cfg(const i4d_config* c) {
    if (!c) return I4D_EINVAL;
    if (c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->d_ff <= 0) return I4D_EINVAL;
    if (c->head_dim != 64 && c->head_dim != 128) return I4D_EINVAL;
    if (c->n_q_heads % c->n_kv_heads != 0 || c->n_q_heads / c->n_kv_heads > 16) return I4D_EINVAL;
    if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.0)) return I4D_EINVAL;
    if (c->exec_mode < 0 || c->exec_mode > 2) return I4D_EINVAL;
    return I4D_OK;
}

int validate_layer(const i4d_config* c, const i4d_layer* L) {
    if (!L || !L->attn_norm || !L->ffn_norm) return I4D_EINVAL;
    if (!aligned(L->attn_norm, 2) || !aligned(L->ffn_norm, 2)) return I4D_EALIGN;
    const int D = c->d_model, qw = c->n_q_heads * c->head_dim, kvw = c->n_kv_heads * c->head_dim, F = c->d_ff;
    const int dt = L->wq.dtype, g = L->wq.group;
    int rc;
    if ((rc = validate_mat(&L->wq, qw, D, dt, g))) return rc;
    if ((rc = validate_mat(&L->wk, kvw, D, dt, g))) return rc;
    if ((rc = validate_mat(&L->wv, kvw, D, dt, g))) return rc;
    if ((rc = validate_mat(&L->wo, D, qw, dt, g))) return rc;
    if ((rc = validate_mat(&L->wg, F, D, dt, g))) return rc;
    if ((rc = validate_mat(&L->wu, F, D, dt, g))) return rc;
    if ((rc = validate_mat(&L->wd, D, F, dt, g))) return rc;
    return I4D_OK;
}

int validate_kv(const i4d_config* c, const i4d_kv* kv, int max_pos) {
    (void)c;
    if (!kv || !kv->k || !kv->v) return I4D_EINVAL;
    if (kv->capacity <= 0 || kv->capacity % 16 != 0) return I4D_EINVAL;
    if (!aligned(kv->k, 16) || !aligned(kv->v, 16)) return I4D_EALIGN;
    if (kv->pages) {
        if (kv->page_size <= 0 || kv->page_size % 16 != 0 || kv->capacity % kv->page_size != 0 || kv->n_pages < 1)
            return I4D_EINVAL;
        if (!aligned(kv->pages, 4)) return I4D_EALIGN;
    }
    if (max_pos < 0 || max_pos >= kv->capacity) return I4D_ERANGE;
    return I4D_OK;
}

int validate_ws(void* ws, size_t ws_bytes, size_t need) {
    if (!ws) return I4D_EWORKSPACE;
    if (!aligned(ws, 256)) return I4D_EALIGN;
    if (ws_bytes < need) return I4D_EWORKSPACE;
    return I4D_OK;
}

DevMat dev_mat(const i4d_mat& m) {
    DevMat d;
    d.data = (const uint8_t*)m.data;
    d.scales = (const uint16_t*)m.scales;
    d.n = m.n; d.k = m.k; d.group = m.group;
    d.ngroups = (m.dtype == I4D_WEIGHT_INT4) ? (m.k + m.group - 1) / m.group : 0;
    return d;
}

int pick_fmt(const i4d_mat& m) {
    if (m.dtype == I4D_WEIGHT_INT4)
        return (m.k % 512 == 0 && is_pow2(m.group) && m.group >= 32 && (m.k / m.group) % 2 == 0 && aligned(m.scales, 4))
                   ? FMT_INT4_FAST : FMT_INT4_GEN;
    return (m.k % 128 == 0) ? FMT_BF16_FAST : FMT_BF16_GEN;
}

// One format for a task that streams several matrices: the fast int4 path
// needs every one of them to qualify.
int pick_fmt(const i4d_mat& a, const i4d_mat& b, const i4d_mat* c = nullptr) {
    const int f = pick_fmt(a);
    if (f == FMT_INT4_FAST && (pick_fmt(b) != FMT_INT4_FAST || (c && pick_fmt(*c) != FMT_INT4_FAST)))
        return FMT_INT4_GEN;
    return f;
}

int unit_w(int fmt) {
    switch (fmt) {
        case FMT_INT4_FAST: return FmtT<FMT_INT4_FAST>::UNIT_W;
        case FMT_INT4_GEN: return FmtT<FMT_INT4_GEN>::UNIT_W;
        case FMT_BF16_FAST: return FmtT<FMT_BF16_FAST>::UNIT_W;
        default: return FmtT<FMT_BF16_GEN>::UNIT_W;
    }
}

int nb_slot(int batch) { return batch <= 1 ? 1 : batch <= 2 ? 2 : batch <= 4 ? 4 : 8; }
int maxj_of(int nb) { return nb <= 2 ? MaxJ<1>::v : MaxJ<4>::v; }

// Fill pass geometry: at most `cap_pairs` pairs per pass (0: no cap), and never
// more pairs per workgroup than keeps every slot within MAXJ runs.
// young: the younger waves' share in percent (see wave_cut); the best value
// was measured per matrix shape.
void plan_passes(GemvTask& t, int fmt, int nb, int nwg, int cap_pairs, int nt = GEMV_NT, int young = 50) {
    const int S = (t.k + unit_w(fmt) - 1) / unit_w(fmt);
    const int maxj = maxj_of(nb);
    t.young = young;
    int ppw = (t.total_pairs + nwg - 1) / nwg;
    while (ppw > 1 && gemv_max_runs(ppw, S, nt / 64, young) > maxj) --ppw;
    long long pp = (long long)ppw * nwg;
    if (cap_pairs > 0 && pp > cap_pairs) pp = cap_pairs;
    if (pp > t.total_pairs) pp = t.total_pairs;
    if (pp < 1) pp = 1;
    // with pp pairs per pass a workgroup gets at most ceil(pp / nwg) <= ppw pairs
    t.pass_pairs = (int)pp;
    t.npasses = (t.total_pairs + t.pass_pairs - 1) / t.pass_pairs;
}

GemvTask make_task(int kind, const i4d_mat* a, const i4d_mat* b, const i4d_mat* c, int head_dim) {
    GemvTask t;
    memset(&t, 0, sizeof(t));
    t.kind = kind;
    t.a = dev_mat(*a);
    t.b = b ? dev_mat(*b) : t.a;
    t.c = c ? dev_mat(*c) : t.a;
    t.k = a->k;
    t.pitch_k = a->k;
    t.log2_group = (a->dtype == I4D_WEIGHT_INT4) ? ilog2(a->group) : 0;
    t.head_dim = head_dim;
    if (kind == KIND_ADJ) t.total_pairs = (a->n + 1) / 2;
    else if (kind == KIND_TWO) t.total_pairs = a->n;
    else t.total_pairs = (a->n + b->n + c->n) / 2;
    return t;
}

// Every kernel is launched only if it runs without scratch memory: a
// private segment would mean the compiler put registers or arrays in slow
// per-lane memory (and that the dispatch must provide it).  The build checks
// every kernel's code object for one; this is the run-time check of the
// same, once per kernel and device (a host-side cache).
struct KernAttr { const void* fn; int dev; size_t lds; bool scratch_free; };
KernAttr g_kern_attr[512];
int g_kern_attr_n = 0;

KernAttr* kern_attr(const void* fn) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    for (int i = 0; i < g_kern_attr_n; ++i)
        if (g_kern_attr[i].fn == fn && g_kern_attr[i].dev == dev) return &g_kern_attr[i];
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, fn) != hipSuccess) return nullptr;
    if (g_kern_attr_n >= 512) return nullptr;
    g_kern_attr[g_kern_attr_n] = KernAttr{fn, dev, 0, fa.localSizeBytes == 0};
    return &g_kern_attr[g_kern_attr_n++];
}

// I4D_OK, or I4D_EUNSUPPORTED for a kernel that needs scratch, or I4D_EHIP.
template <class K>
int scratch_free(K kernel) {
    const KernAttr* a = kern_attr((const void*)kernel);
    if (!a) return I4D_EHIP;
    return a->scratch_free ? I4D_OK : I4D_EUNSUPPORTED;
}

// The scratch check, then the kernel's dynamic-LDS limit raised to `bytes`
// (the attribute only ever grows).
template <class K>
int set_lds(K kernel, size_t bytes) {
    KernAttr* a = kern_attr((const void*)kernel);
    if (!a) return I4D_EHIP;
    if (!a->scratch_free) return I4D_EUNSUPPORTED;
    if (a->lds >= bytes) return I4D_OK;
    if (hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
        return I4D_EHIP;
    a->lds = bytes;
    return I4D_OK;
}

constexpr size_t LDS_LIMIT = 160 * 1024;

// ---------------------------------------------------------------- typed launchers
#define I4D_DISPATCH(FMTV, NBV, CALL)                                                         \
    switch (FMTV) {                                                                           \
        case FMT_INT4_FAST: switch (NBV) { case 1: CALL(FMT_INT4_FAST, 1); case 2: CALL(FMT_INT4_FAST, 2); \
                                           case 4: CALL(FMT_INT4_FAST, 4); default: CALL(FMT_INT4_FAST, 8); } \
        case FMT_INT4_GEN: switch (NBV) { case 1: CALL(FMT_INT4_GEN, 1); case 2: CALL(FMT_INT4_GEN, 2); \
                                          case 4: CALL(FMT_INT4_GEN, 4); default: CALL(FMT_INT4_GEN, 8); } \
        case FMT_BF16_FAST: switch (NBV) { case 1: CALL(FMT_BF16_FAST, 1); case 2: CALL(FMT_BF16_FAST, 2); \
                                           case 4: CALL(FMT_BF16_FAST, 4); default: CALL(FMT_BF16_FAST, 8); } \
        default: switch (NBV) { case 1: CALL(FMT_BF16_GEN, 1); case 2: CALL(FMT_BF16_GEN, 2);     \
                                case 4: CALL(FMT_BF16_GEN, 4); default: CALL(FMT_BF16_GEN, 8); } \
    }

// ---------------------------------------------------------------- launch timing
// Measurement aid behind i4d_launch_timing_start/stop.  A TimeScope of the
// selected kind arms the next library kernel launch (launch_k), which then
// goes out through hipExtLaunchKernel with a start and a stop event: the
// runtime stamps them with the kernel's own start and end, so no extra
// packet sits between kernels.
struct LaunchTiming {
    int kind = 0, cap = 0, n = 0;
    bool armed = false;
    std::vector<hipEvent_t> ev;          // 2 per launch: start, stop
};
LaunchTiming g_timing;

struct TimeScope {
    explicit TimeScope(int kind) { g_timing.armed = (g_timing.kind == kind); }
    ~TimeScope() { g_timing.armed = false; }
};

// The timed slot for the launch about to be made (-1: not timed).
int take_timing_slot() {
    if (!g_timing.armed || g_timing.n >= g_timing.cap) return -1;
    g_timing.armed = false;
    return g_timing.n++;
}

template <class F, class... A>
void launch_k(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, A... args) {
    const int slot = take_timing_slot();
    hipEvent_t e0 = slot >= 0 ? g_timing.ev[2 * slot] : nullptr;
    hipEvent_t e1 = slot >= 0 ? g_timing.ev[2 * slot + 1] : nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, e0, e1, 0u, args...);
}

template <int FMT, int NB>
int launch_rows_t(const GemvTask& t, int nwg, const float* x, int x_stride, int nb, const uint16_t* gain, float eps,
                  float* y, const float* resid, hipStream_t s) {
    const size_t lds = gemv_lds_bytes<FMT, NB, PREC_STD>(t.k);
    if (lds > LDS_LIMIT) return I4D_EUNSUPPORTED;
    if (const int rc_ = set_lds(k_gemv_rows<FMT, NB>, lds)) return rc_;
    launch_k(k_gemv_rows<FMT, NB>, dim3(nwg), dim3(GEMV_NT), lds, s, t, x, x_stride, nb, gain, eps, y, resid);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

template <int FMT, int NB>
int launch_swiglu_t(const GemvTask& t, int nwg, const float* x, int nb, const uint16_t* gain, float eps, float* act, hipStream_t s) {
    const size_t lds = gemv_lds_bytes<FMT, NB, PREC_STD>(t.k);
    if (lds > LDS_LIMIT) return I4D_EUNSUPPORTED;
    if (const int rc_ = set_lds(k_gemv_swiglu<FMT, NB>, lds)) return rc_;
    launch_k(k_gemv_swiglu<FMT, NB>, dim3(nwg), dim3(GEMV_NT), lds, s, t, x, nb, gain, eps, act);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

// page map of a cache (pages == nullptr: contiguous)
KvMap kv_map(const i4d_kv* kv) {
    if (!kv->pages) return KvMap{nullptr, 0, 0, 0};
    return KvMap{kv->pages, kv->page_size / 16, kv->n_pages, kv->capacity / kv->page_size};
}

template <int FMT, int NB>
int launch_qkv_t(const GemvTask& t, int nwg, const float* x, int nb, const uint16_t* gain, float eps, const int* pos, int max_pos,
                 float* q, const i4d_kv* kv, uint16_t* kvn, int hq, int hkv, double base, int* status, int kvb, hipStream_t s) {
    const size_t lds = gemv_lds_bytes<FMT, NB, PREC_QKV>(t.k);
    if (lds > LDS_LIMIT) return I4D_EUNSUPPORTED;
    if (const int rc_ = set_lds(k_gemv_qkv<FMT, NB>, lds)) return rc_;
    launch_k(k_gemv_qkv<FMT, NB>, dim3(nwg), dim3(GEMV_NT), lds, s, t, x, nb, gain, eps, pos, max_pos, q,
                       kv->k, kv->v, kvn, kv->capacity, hq, hkv, base, status, kvb, kv_map(kv));
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

template <int FMT, int NB>
int launch_lm_t(const GemvTask& t, int nwg, const float* h, int nb, u64* wg_keys, int32_t* tok, float* mx, const Sampler& smp,
                hipStream_t s) {
    if constexpr (!FmtT<FMT>::INT4) {
        return I4D_EUNSUPPORTED;
    } else {
        const size_t lds = gemv_lds_bytes<FMT, NB, PREC_STD>(t.k) + (size_t)GEMV_NT * 12;
        if (lds > LDS_LIMIT) return I4D_EUNSUPPORTED;
        if (const int rc_ = set_lds(k_lm_head<FMT, NB>, lds)) return rc_;
        if (const int rc_ = scratch_free(k_lm_finalize)) return rc_;
        launch_k(k_lm_head<FMT, NB>, dim3(nwg), dim3(GEMV_NT), lds, s, t, h, nb, wg_keys, smp);
        hipLaunchKernelGGL(k_lm_finalize, dim3(1), dim3(256), 0, s, (const u64*)wg_keys, nwg, MAX_BATCH, nb, tok, mx);
        return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
    }
}

int launch_rows(int fmt, int nb, const GemvTask& t, int nwg, const float* x, int x_stride, int bn, const uint16_t* gain,
                float eps, float* y, const float* resid, hipStream_t s) {
#define CALL(F, N) return launch_rows_t<F, N>(t, nwg, x, x_stride, bn, gain, eps, y, resid, s)
    I4D_DISPATCH(fmt, nb, CALL)
#undef CALL
}
size_t rows_lds_bytes(int fmt, int nb, int K) {
#define CALL(F, N) return gemv_lds_bytes<F, N, PREC_STD>(K)
    I4D_DISPATCH(fmt, nb, CALL)
#undef CALL
}

// y = resid + W x through k_gemv_rows, in `c` equal K-chunks when the staged
// activations of the whole row would not fit in LDS (large K with several
// sequences): chunk 0 adds resid, every later chunk adds onto y in place (the
// same thread reads and writes each element), so the sum order is fixed.
int chunk_count(int fmt, int nb, int K, int group) {
    if (rows_lds_bytes(fmt, nb, K) <= LDS_LIMIT) return 1;
    if (fmt != FMT_INT4_FAST && fmt != FMT_BF16_FAST) return 0;
    for (int c = 2; c <= 16; ++c) {
        if (K % c) continue;
        const int kc = K / c;
        if (kc % unit_w(fmt)) continue;
        if (fmt == FMT_INT4_FAST && (kc % group || (kc / group) % 2)) continue;
        if (rows_lds_bytes(fmt, nb, kc) <= LDS_LIMIT) return c;
    }
    return 0;
}

size_t qkv_lds_bytes(int fmt, int nb, int K) {
#define CALL(F, N) return gemv_lds_bytes<F, N, PREC_QKV>(K)
    I4D_DISPATCH(fmt, nb, CALL)
#undef CALL
}

// Host check, before anything is enqueued, that every phase of a layer fits
// the per-workgroup LDS at this batch (the row GEMVs may split K).
int phases_fit(const i4d_layer* L, int batch) {
    const int nb = nb_slot(batch);
    if (qkv_lds_bytes(pick_fmt(L->wq, L->wk, &L->wv), nb, L->wq.k) > LDS_LIMIT) return I4D_EUNSUPPORTED;
    if (rows_lds_bytes(pick_fmt(L->wg, L->wu), nb, L->wg.k) > LDS_LIMIT) return I4D_EUNSUPPORTED;
    if (chunk_count(pick_fmt(L->wo), nb, L->wo.k, L->wo.group) == 0) return I4D_EUNSUPPORTED;
    if (chunk_count(pick_fmt(L->wd), nb, L->wd.k, L->wd.group) == 0) return I4D_EUNSUPPORTED;
    return I4D_OK;
}

int launch_rows_chunked(int fmt, int nb, const GemvTask& t, int nwg, const float* x, int x_stride, int bn, float* y,
                        const float* resid, int young, hipStream_t s) {
    const int c = chunk_count(fmt, nb, t.k, t.a.group);
    if (c == 0) return I4D_EUNSUPPORTED;
    const int kc = t.k / c;
    for (int i = 0; i < c; ++i) {
        GemvTask tc = t;
        tc.k = kc;
        if (fmt == FMT_INT4_FAST) {
            tc.a.data += (size_t)i * (kc >> 1);
            tc.a.scales += (size_t)i * (kc / t.a.group);
        } else if (fmt == FMT_BF16_FAST) {
            tc.a.data += (size_t)i * kc * 2;
        }
        tc.b = tc.a; tc.c = tc.a;
        plan_passes(tc, fmt, nb, nwg, 0, GEMV_NT, young);
        const int rc = launch_rows(fmt, nb, tc, nwg, x + (size_t)i * kc, x_stride, bn, nullptr, 0.f, y, i == 0 ? resid : y, s);
        if (rc) return rc;
    }
    return I4D_OK;
}

int launch_swiglu(int fmt, int nb, const GemvTask& t, int nwg, const float* x, int bn, const uint16_t* gain, float eps, float* act,
                  hipStream_t s) {
#define CALL(F, N) return launch_swiglu_t<F, N>(t, nwg, x, bn, gain, eps, act, s)
    I4D_DISPATCH(fmt, nb, CALL)
#undef CALL
}
int launch_qkv(int fmt, int nb, const GemvTask& t, int nwg, const float* x, int bn, const uint16_t* gain, float eps,
               const int* pos, int max_pos, float* q, const i4d_kv* kv, uint16_t* kvn, int hq, int hkv, double base, int* status,
               int kvb, hipStream_t s) {
#define CALL(F, N) return launch_qkv_t<F, N>(t, nwg, x, bn, gain, eps, pos, max_pos, q, kv, kvn, hq, hkv, base, status, kvb, s)
    I4D_DISPATCH(fmt, nb, CALL)
#undef CALL
}
int launch_lm(int fmt, int nb, const GemvTask& t, int nwg, const float* h, int bn, u64* keys, int32_t* tok, float* mx,
              const Sampler& smp, hipStream_t s) {
#define CALL(F, N) return launch_lm_t<F, N>(t, nwg, h, bn, keys, tok, mx, smp, s)
    I4D_DISPATCH(fmt, nb, CALL)
#undef CALL
}

// attention split plan
void plan_attention(const i4d_config* c, int B, int max_pos, int& nsplit, int& T) {
    const int nk = max_pos + 1;
    int want = (num_cus() + B * c->n_kv_heads - 1) / (B * c->n_kv_heads);
    want = std::max(1, std::min(want, NSPLIT_MAX));
    T = (nk + want - 1) / want;
    T = std::max(16, ((T + 15) / 16) * 16);      // whole 16-position cache tiles
    nsplit = (nk + T - 1) / T;
}

// Attention arguments for layer region R (kvn = nullptr: the cache already
// holds every attended key, as for the attention test hook).
AttnArgs attn_args(const i4d_config* c, int B, const float* q, const i4d_kv* kv, const uint16_t* kvn, const int* pos,
                   int max_pos, float* o, char* ws, const WsLayout& W, const char* R, int kvb = 1) {
    AttnArgs a;
    a.kvb = kvb;
    a.q = q; a.kc = kv->k; a.vc = kv->v; a.kvn = kvn; a.pos = pos;
    a.cap = kv->capacity; a.hq = c->n_q_heads; a.hkv = c->n_kv_heads; a.batch = B; a.max_pos = max_pos;
    plan_attention(c, B, max_pos, a.nsplit, a.T);
    a.pstride = W.pstride;
    a.qscale = (float)(1.4426950408889634 / sqrt((double)c->head_dim));
    a.pm = (float*)(R + W.pm); a.pl = (float*)(R + W.pl); a.po = (float*)(R + W.po);
    a.cnt = (int*)(ws + WS_CNT);
    a.o = o;
    a.pg = kv_map(kv);
    a.status = (int*)(ws + WS_STATUS);
    return a;
}

template <int HD, bool PAGED>
int launch_attention_t(const AttnArgs& a, hipStream_t s) {
    const int items = a.batch * a.hkv * a.nsplit;
    const size_t lds = attn_lds_bytes<HD, ATTN_NT>();
    if (const int rc_ = set_lds(k_attention<HD, PAGED>, lds)) return rc_;
    launch_k(k_attention<HD, PAGED>, dim3(items), dim3(ATTN_NT), lds, s, a);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

int launch_attention(const AttnArgs& a, int hd, hipStream_t s) {
    const bool paged = a.pg.pages != nullptr;
    if (hd == 128) return paged ? launch_attention_t<128, true>(a, s) : launch_attention_t<128, false>(a, s);
    return paged ? launch_attention_t<64, true>(a, s) : launch_attention_t<64, false>(a, s);
}

// ---------------------------------------------------------------- batched (MFMA) path
// Batches of 9..32 sequences (padded to 16 or 32 MFMA columns).  Each
// projection is a staging launch (norm, fp16 conversion)
// followed by the MFMA GEMM with the same epilogue as the matrix-vector path.
bool mfma_mat_ok(const i4d_mat& m) {
    return m.dtype == I4D_WEIGHT_INT4 && m.k % 256 == 0 && (m.group == 128 || m.group == 256) && (m.k / m.group) % 2 == 0 &&
           aligned(m.scales, 4) && aligned(m.data, 16);
}
int nb_mfma(int batch) { return batch <= 16 ? 16 : 32; }

struct MfmaPlan { int tiles, rbs, kb, spb, nsteps, nwg; };

// Row blocks of 8*RT tiles; the K axis is split over workgroups (at least two
// LDS chunks per block) up to one workgroup per compute unit.  (Where the LDS
// lets two workgroups share a CU, grids with more row blocks than CUs run in
// one round; splitting K further costs more in partial sums than it gains.)
MfmaPlan mfma_plan(int total_pairs, int K, int nb, int prec, bool split) {
    MfmaPlan p;
    // the kernel's own geometry for this column count and activation precision
    const int tb = nb == 16 ? (prec == 1 ? MfmaGeo<16, 1>::TB : MfmaGeo<16, 2>::TB)
                            : (prec == 1 ? MfmaGeo<32, 1>::TB : MfmaGeo<32, 2>::TB);
    const int sc = nb == 16 ? (prec == 1 ? MfmaGeo<16, 1>::SC : MfmaGeo<16, 2>::SC)
                            : (prec == 1 ? MfmaGeo<32, 1>::SC : MfmaGeo<32, 2>::SC);
    const int slots = num_cus();
    p.tiles = (total_pairs + 7) / 8;
    p.rbs = (p.tiles + tb - 1) / tb;
    p.nsteps = K / 128;
    int kb = 1;
    if (split && p.rbs < slots) {
        kb = std::max(1, slots / p.rbs);          // within one round of workgroups
        kb = std::min(kb, std::max(1, p.nsteps / (2 * sc)));
    }
    p.spb = (p.nsteps + kb - 1) / kb;
    p.spb = (p.spb + sc - 1) / sc * sc;             // K blocks start on a chunk (an even step, an even group)
    p.kb = (p.nsteps + p.spb - 1) / p.spb;
    p.nwg = p.rbs * p.kb;
    return p;
}
size_t mfma_part_bytes(const MfmaPlan& p, int nb) { return p.kb > 1 ? (size_t)p.tiles * p.kb * nb * 16 * 4 : 0; }

// Scratch of one batched phase: staged activations (up to two planes),
// partial sums, validated positions and the RoPE table.
struct MfmaScratch { size_t xs, part, posv, cs, xsc, total; };
MfmaScratch mfma_scratch(int kmax, int nb, size_t part_bytes, int hd) {
    MfmaScratch m;
    size_t off = 0;
    auto take = [&](size_t b) { size_t o = off; off = align256(off + b); return o; };
    m.xs = take((size_t)2 * nb * kmax * 2);
    m.part = take(part_bytes);
    m.posv = take((size_t)nb * 4);
    m.cs = take((size_t)nb * (hd / 2) * 8);
    m.xsc = take((size_t)nb * 4);
    m.total = off;
    return m;
}
MfmaScratch layer_scratch(const i4d_config* c, int nb) {
    const int D = c->d_model, qw = c->n_q_heads * c->head_dim, kvw = c->n_kv_heads * c->head_dim, F = c->d_ff;
    size_t part = 0;
    part = std::max(part, mfma_part_bytes(mfma_plan((qw + 2 * kvw) / 2, D, nb, 2, true), nb));
    part = std::max(part, mfma_part_bytes(mfma_plan((D + 1) / 2, qw, nb, 1, true), nb));
    part = std::max(part, mfma_part_bytes(mfma_plan(F, D, nb, 1, true), nb));
    part = std::max(part, mfma_part_bytes(mfma_plan((D + 1) / 2, F, nb, 1, true), nb));
    return mfma_scratch(std::max(std::max(D, qw), F), nb, part, c->head_dim);
}

size_t layer_scratch_bytes(const i4d_config* c, int nb) { return layer_scratch(c, nb).total; }

MfmaTask mfma_task(const GemvTask& t, const MfmaPlan& p, char* base, const MfmaScratch& S, int* cnt, int batch, int group) {
    MfmaTask m;
    memset(&m, 0, sizeof(m));
    m.t = t;
    m.xs = (const uint32_t*)(base + S.xs);
    m.xscale = (const float*)(base + S.xsc);
    m.part = (float*)(base + S.part);
    m.cnt = cnt;
    m.tiles = p.tiles; m.kb = p.kb; m.spb = p.spb; m.nsteps = p.nsteps;
    m.gshift = ilog2(group) - 7;
    m.nb = batch;
    return m;
}

int mfma_stage(int prec, int nb, const float* x, int stride, int batch, int K, const uint16_t* gain, float eps, char* base,
               const MfmaScratch& S, const int* pos, int max_pos, int cap, int hd, double rope_base, bool rope, int* status,
               hipStream_t s) {
    uint32_t* xs = (uint32_t*)(base + S.xs);
    int* posv = rope ? (int*)(base + S.posv) : nullptr;
    float2* cs = rope ? (float2*)(base + S.cs) : nullptr;
    float* xsc = (float*)(base + S.xsc);
    if (const int rc_ = scratch_free(prec == 2 ? k_mfma_stage<2> : k_mfma_stage<1>)) return rc_;
    if (prec == 2)
        hipLaunchKernelGGL(k_mfma_stage<2>, dim3(nb), dim3(256), 0, s, x, stride, batch, nb, K, gain, eps, xs, pos, max_pos,
                           cap, hd, rope_base, posv, cs, status, xsc);
    else
        hipLaunchKernelGGL(k_mfma_stage<1>, dim3(nb), dim3(256), 0, s, x, stride, batch, nb, K, gain, eps, xs, pos, max_pos,
                           cap, hd, rope_base, posv, cs, status, xsc);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

template <class Kern, class... A>
int launch_mfma(Kern kernel, size_t lds, const MfmaPlan& p, hipStream_t s, A... args) {
    if (lds > LDS_LIMIT) return I4D_EUNSUPPORTED;
    if (p.kb > 1 && p.rbs > WS_MAX_MCNT) return I4D_EUNSUPPORTED;
    if (const int rc_ = set_lds(kernel, lds)) return rc_;
    launch_k(kernel, dim3(p.nwg), dim3(MfmaGeo<16, 1>::NT), lds, s, args...);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

int mfma_rows(int nb, const MfmaTask& m, const MfmaPlan& p, float* y, const float* resid, hipStream_t s) {
    return nb == 16 ? launch_mfma(k_mfma_rows<16>, MfmaGeo<16, 1>::LDS_B, p, s, m, y, resid)
                    : launch_mfma(k_mfma_rows<32>, MfmaGeo<32, 1>::LDS_B, p, s, m, y, resid);
}

bool mfma_layer_ok(const i4d_config* c, const i4d_layer* L) {
    const i4d_mat* m[7] = {&L->wq, &L->wk, &L->wv, &L->wo, &L->wg, &L->wu, &L->wd};
    for (int i = 0; i < 7; ++i)
        if (!mfma_mat_ok(*m[i])) return false;
    return c->d_model % 256 == 0 && c->d_ff % 256 == 0 && (c->n_q_heads * c->head_dim) % 256 == 0;
}

// One layer for 9..32 sequences: staging + MFMA GEMM per projection, the
// split-K attention in between (which handles any batch).
int run_layer_mfma(const i4d_config* c, const i4d_layer* L, int B, const float* x_in, float* x_out, const i4d_kv* kv,
                   const int* pos, int max_pos, char* ws, const WsLayout& W, char* R, hipStream_t s, int kvb) {
    const int nb = nb_mfma(B), hd = c->head_dim;
    const int D = c->d_model, qw = c->n_q_heads * hd, F = c->d_ff, g = L->wq.group;
    int* status = (int*)(ws + WS_STATUS);
    int* cnt = (int*)(ws + WS_MCNT);
    char* base = ws + W.mfma;
    const MfmaScratch S = layer_scratch(c, nb);
    uint16_t* kvn = (uint16_t*)(R + W.kvn);
    float* q = (float*)(R + W.q);
    float* o = (float*)(R + W.o);
    float* y = (float*)(R + W.y);
    float* act = (float*)(R + W.act);
    int rc;

    if ((rc = mfma_stage(2, nb, x_in, D, B, D, L->attn_norm, c->rms_eps, base, S, pos, max_pos, kv->capacity, hd, c->rope_base,
                         true, status, s)))
        return rc;
    const GemvTask tq = make_task(KIND_QKV, &L->wq, &L->wk, &L->wv, hd);
    const MfmaPlan pq = mfma_plan(tq.total_pairs, D, nb, 2, true);
    const MfmaTask mq = mfma_task(tq, pq, base, S, cnt, B, g);
    const int* posv = (const int*)(base + S.posv);
    const float2* cs = (const float2*)(base + S.cs);
    {
        TimeScope ts(I4D_TIME_QKV);
        rc = nb == 16 ? launch_mfma(k_mfma_qkv<16>, MfmaGeo<16, 2>::LDS_B, pq, s, mq, q, kv->k, kv->v, kvn, posv, cs, kv->capacity,
                                    c->n_q_heads, c->n_kv_heads, kvb, kv_map(kv), status)
                      : launch_mfma(k_mfma_qkv<32>, MfmaGeo<32, 2>::LDS_B, pq, s, mq, q, kv->k, kv->v, kvn, posv, cs, kv->capacity,
                                    c->n_q_heads, c->n_kv_heads, kvb, kv_map(kv), status);
    }
    if (rc) return rc;
    {
        TimeScope ts(I4D_TIME_ATTENTION);
        rc = launch_attention(attn_args(c, B, q, kv, kvn, pos, max_pos, o, ws, W, R, kvb), hd, s);
    }
    if (rc) return rc;

    if ((rc = mfma_stage(1, nb, o, qw, B, qw, nullptr, 0.f, base, S, nullptr, 0, 0, hd, 0.0, false, status, s))) return rc;
    const GemvTask to = make_task(KIND_ADJ, &L->wo, nullptr, nullptr, hd);
    const MfmaPlan po = mfma_plan(to.total_pairs, qw, nb, 1, true);
    {
        TimeScope ts(I4D_TIME_WO);
        rc = mfma_rows(nb, mfma_task(to, po, base, S, cnt, B, g), po, y, x_in, s);
    }
    if (rc) return rc;

    if ((rc = mfma_stage(1, nb, y, D, B, D, L->ffn_norm, c->rms_eps, base, S, nullptr, 0, 0, hd, 0.0, false, status, s))) return rc;
    const GemvTask tg = make_task(KIND_TWO, &L->wg, &L->wu, nullptr, hd);
    const MfmaPlan pg = mfma_plan(tg.total_pairs, D, nb, 1, true);
    const MfmaTask mg = mfma_task(tg, pg, base, S, cnt, B, g);
    {
        TimeScope ts(I4D_TIME_GATE_UP);
        rc = nb == 16 ? launch_mfma(k_mfma_swiglu<16>, MfmaGeo<16, 1>::LDS_B, pg, s, mg, act)
                      : launch_mfma(k_mfma_swiglu<32>, MfmaGeo<32, 1>::LDS_B, pg, s, mg, act);
    }
    if (rc) return rc;

    if ((rc = mfma_stage(1, nb, act, F, B, F, nullptr, 0.f, base, S, nullptr, 0, 0, hd, 0.0, false, status, s))) return rc;
    const GemvTask td = make_task(KIND_ADJ, &L->wd, nullptr, nullptr, hd);
    const MfmaPlan pd = mfma_plan(td.total_pairs, F, nb, 1, true);
    TimeScope ts(I4D_TIME_DOWN);
    return mfma_rows(nb, mfma_task(td, pd, base, S, cnt, B, g), pd, x_out, y, s);
}

// ---------------------------------------------------------------- prompt prefill
// GEMM kernels of the prefill path (prefill.h), one per epilogue.  The
// wide-tile ones are built for the waves per SIMD their tile size runs at.
__global__ void __launch_bounds__(PF_NT) __attribute__((amdgpu_waves_per_eu(PF_BM_ROWS == 128 ? 1 : 2, PF_BM_ROWS == 128 ? 1 : 2)))
k_pf_rows(PfTask g, float* y, const float* resid) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    EpiRows<false> ep{y, resid, g.t.a.n, g.ntok};
    pf_gemm<KIND_ADJ, 1, PF_BM_ROWS>(g, lds, ep);
}

__global__ void __launch_bounds__(PF_NT) __attribute__((amdgpu_waves_per_eu(PF_BM_WIDE == 128 ? 1 : 2, PF_BM_WIDE == 128 ? 1 : 2)))
k_pf_swiglu(PfTask g, float* act) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    EpiSwiGLU<false> ep{act, g.t.a.n, g.ntok};
    pf_gemm<KIND_TWO, 1, PF_BM_WIDE>(g, lds, ep);
}

// q (fp32, RoPE applied) to its buffer, bf16 k/v appended at each token's slot
__global__ void __launch_bounds__(PF_NT) k_pf_qkv(PfTask g, float* q, uint16_t* kc, uint16_t* vc, const int* posv,
                                                  const float2* cs, int cap, int hq, int hkv, KvMap pgm, int* status) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    EpiQKV<false> ep{q, kc, vc, nullptr, posv, cs, cap, hq, hkv, g.t.head_dim, g.ntok, 0, pgm, status};
    int mt, nt, kss;
    pf_tile(g, mt, nt, kss);
    // q rows from the fp16 value plane alone (q enters attention as bf16
    // high + low parts); k and v rows, rounded to bf16 into the cache, also
    // take the remainder plane
    if (nt < g.nlo) pf_gemm<KIND_QKV, 1, PF_BM_QKV>(g, lds, ep);
    else pf_gemm<KIND_QKV, 2, PF_BM_QKV>(g, lds, ep);
}

// Tiles of one prefill GEMM; the K axis is split (adjacent-row tasks only)
// while the tiles fill fewer than two workgroups per compute unit, keeping at
// least 8 steps per split.
struct PfPlan { int mtiles, ntiles, ks, spk, nsteps, nwg; };
PfPlan pf_plan(int total_pairs, int K, int ntok, bool split, int bm) {
    PfPlan p;
    p.mtiles = (ntok + bm - 1) / bm;
    p.ntiles = (total_pairs + PF_PAIRS - 1) / PF_PAIRS;
    p.nsteps = K / 128;
    const int slots = (bm == 128 ? 1 : 2) * num_cus();   // resident workgroups per CU
    const int base = p.mtiles * p.ntiles;
    int ks = 1;
    if (split && base < slots) ks = std::max(1, std::min(slots / base, p.nsteps / 8));
    p.spk = (p.nsteps + ks - 1) / ks;
    p.ks = (p.nsteps + p.spk - 1) / p.spk;
    p.nwg = base * p.ks;
    return p;
}

// Workspace of i4d_prefill: the status header, then per prompt of T tokens
// (sp = T rounded up to 64) the staged activations (two planes), their
// per-token powers of two, positions and RoPE table, q and the attention
// output, the residual stream, the SwiGLU activations, two layer outputs and
// the split-K partial sums.
struct PfWs { size_t xs, xsc, posv, pos, cs, q, o, y, act, xa, xb, part, total; };
PfWs pf_ws(const i4d_config* c, int T) {
    const size_t sp = (size_t)(T + PF_BM_MAX - 1) / PF_BM_MAX * PF_BM_MAX;
    const size_t D = c->d_model, qw = (size_t)c->n_q_heads * c->head_dim, F = c->d_ff;
    const size_t kmax = std::max(std::max(D, qw), F);
    PfWs w;
    size_t off = WS_HEADER;
    auto take = [&](size_t b) { size_t o = off; off = align256(off + b); return o; };
    w.xs = take(2 * sp * kmax * 2);
    w.xsc = take(sp * 4);
    w.posv = take(sp * 4);
    w.pos = take(sp * 4);
    w.cs = take(sp * (c->head_dim / 2) * 8);
    w.q = take((size_t)T * qw * 4);
    w.o = take((size_t)T * qw * 4);
    w.y = take((size_t)T * D * 4);
    w.act = take((size_t)T * F * 4);
    w.xa = take((size_t)T * D * 4);
    w.xb = take((size_t)T * D * 4);
    size_t part = 0;
    for (int kk = 0; kk < 2; ++kk) {          // the two adjacent-row GEMMs (Wo: K = qw, down: K = F), N = D
        const PfPlan pp = pf_plan((int)((D + 1) / 2), kk == 0 ? (int)qw : (int)F, T, true, PF_BM_ROWS);
        if (pp.ks > 1) part = std::max(part, (size_t)pp.ks * T * D * 4);
    }
    w.part = take(part);
    w.total = off;
    return w;
}

PfTask pf_task(const GemvTask& t, const PfPlan& p, char* ws, const PfWs& W, int T, int group, int rows) {
    PfTask g;
    memset(&g, 0, sizeof(g));
    g.t = t;
    g.xs = (const uint32_t*)(ws + W.xs);
    g.xscale = (const float*)(ws + W.xsc);
    g.part = (float*)(ws + W.part);
    g.sp = (T + PF_BM_MAX - 1) / PF_BM_MAX * PF_BM_MAX;
    g.ntok = T;
    g.nsteps = p.nsteps;
    g.gshift = ilog2(group) - 7;
    g.mtiles = p.mtiles; g.ntiles = p.ntiles; g.ks = p.ks; g.spk = p.spk;
    g.rows = rows;
    return g;
}

template <class Kern, class... A>
int launch_pf(Kern kernel, size_t lds, const PfPlan& p, hipStream_t s, A... args) {
    if (lds > LDS_LIMIT) return I4D_EUNSUPPORTED;
    if (const int rc_ = set_lds(kernel, lds)) return rc_;
    launch_k(kernel, dim3(p.nwg), dim3(PF_NT), lds, s, args...);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

// Adjacent-row GEMM + residual, with the split-K reduction when planned.
int pf_rows(const PfTask& g, const PfPlan& p, float* y, const float* resid, hipStream_t s) {
    int rc;
    if ((rc = launch_pf(k_pf_rows, pf_lds_bytes<1, PF_BM_ROWS>(), p, s, g, y, resid))) return rc;
    if (p.ks == 1) return I4D_OK;
    if ((rc = scratch_free(k_pf_reduce))) return rc;
    const size_t n = (size_t)g.ntok * g.rows;
    const int nblk = (int)std::min<size_t>((n + 255) / 256, (size_t)num_cus() * 8);
    hipLaunchKernelGGL(k_pf_reduce, dim3(nblk), dim3(256), 0, s, (const float*)g.part, p.ks, g.ntok, g.rows, g.xscale, resid, y);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

// Staging of T token rows into the prefill workspace (k_mfma_stage, one
// workgroup per staged row; rows past T are zero-filled).
int pf_stage(int prec, const float* x, int stride, int T, int K, const uint16_t* gain, float eps, char* ws, const PfWs& W,
             int max_pos, int cap, int hd, double rope_base, bool rope, hipStream_t s) {
    const int sp = (T + PF_BM_MAX - 1) / PF_BM_MAX * PF_BM_MAX;
    uint32_t* xs = (uint32_t*)(ws + W.xs);
    int* status = (int*)(ws + WS_STATUS);
    const int* pos = rope ? (const int*)(ws + W.pos) : nullptr;
    int* posv = rope ? (int*)(ws + W.posv) : nullptr;
    float2* cs = rope ? (float2*)(ws + W.cs) : nullptr;
    float* xsc = (float*)(ws + W.xsc);
    if (const int rc_ = scratch_free(prec == 2 ? k_mfma_stage<2> : k_mfma_stage<1>)) return rc_;
    if (prec == 2)
        hipLaunchKernelGGL(k_mfma_stage<2>, dim3(sp), dim3(256), 0, s, x, stride, T, sp, K, gain, eps, xs, pos, max_pos, cap,
                           hd, rope_base, posv, cs, status, xsc);
    else
        hipLaunchKernelGGL(k_mfma_stage<1>, dim3(sp), dim3(256), 0, s, x, stride, T, sp, K, gain, eps, xs, pos, max_pos, cap,
                           hd, rope_base, posv, cs, status, xsc);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

// One layer of a prompt of T tokens at positions pos0 .. pos0 + T - 1.
int run_layer_prefill(const i4d_config* c, const i4d_layer* L, int T, const float* x_in, float* x_out, const i4d_kv* kv,
                      int pos0, char* ws, const PfWs& W, hipStream_t s) {
    const int hd = c->head_dim, D = c->d_model, qw = c->n_q_heads * hd, F = c->d_ff, g = L->wq.group;
    const int max_pos = pos0 + T - 1;
    int* status = (int*)(ws + WS_STATUS);
    float* q = (float*)(ws + W.q);
    float* o = (float*)(ws + W.o);
    float* y = (float*)(ws + W.y);
    float* act = (float*)(ws + W.act);
    int rc;

    if ((rc = pf_stage(2, x_in, D, T, D, L->attn_norm, c->rms_eps, ws, W, max_pos, kv->capacity, hd, c->rope_base, true, s)))
        return rc;
    const GemvTask tq = make_task(KIND_QKV, &L->wq, &L->wk, &L->wv, hd);
    const PfPlan pq = pf_plan(tq.total_pairs, D, T, false, PF_BM_QKV);
    {
        TimeScope ts(I4D_TIME_QKV);
        PfTask gq = pf_task(tq, pq, ws, W, T, g, 0);
        gq.nlo = std::min(pq.ntiles, (tq.a.n >> 1) / PF_PAIRS);      // row blocks holding q pairs only
        rc = launch_pf(k_pf_qkv, pf_lds_bytes<2, PF_BM_QKV>(), pq, s, gq, q, kv->k, kv->v,
                       (const int*)(ws + W.posv), (const float2*)(ws + W.cs), kv->capacity, c->n_q_heads, c->n_kv_heads,
                       kv_map(kv), status);
    }
    if (rc) return rc;
    {
        PfAttnArgs a;
        a.q = q; a.kc = kv->k; a.vc = kv->v; a.o = o;
        a.ntok = T; a.pos0 = pos0; a.cap = kv->capacity; a.hq = c->n_q_heads; a.hkv = c->n_kv_heads;
        a.nqb = (T + 15) / 16;
        a.qscale = (float)(1.4426950408889634 / std::sqrt((double)hd));
        a.pg = kv_map(kv);
        a.status = status;
        const int nwg = (a.hq * a.nqb + 3) / 4;
        auto kern = hd == 128 ? k_pf_attn<128> : k_pf_attn<64>;
        if ((rc = scratch_free(kern))) return rc;
        TimeScope ts(I4D_TIME_ATTENTION);
        launch_k(kern, dim3(nwg), dim3(256), 0, s, a);
        if (hipGetLastError() != hipSuccess) return I4D_EHIP;
    }

    if ((rc = pf_stage(1, o, qw, T, qw, nullptr, 0.f, ws, W, 0, 0, hd, 0.0, false, s))) return rc;
    const GemvTask to = make_task(KIND_ADJ, &L->wo, nullptr, nullptr, hd);
    const PfPlan po = pf_plan(to.total_pairs, qw, T, true, PF_BM_ROWS);
    {
        TimeScope ts(I4D_TIME_WO);
        rc = pf_rows(pf_task(to, po, ws, W, T, g, D), po, y, x_in, s);
    }
    if (rc) return rc;

    if ((rc = pf_stage(1, y, D, T, D, L->ffn_norm, c->rms_eps, ws, W, 0, 0, hd, 0.0, false, s))) return rc;
    const GemvTask tg = make_task(KIND_TWO, &L->wg, &L->wu, nullptr, hd);
    const PfPlan pg = pf_plan(tg.total_pairs, D, T, false, PF_BM_WIDE);
    {
        TimeScope ts(I4D_TIME_GATE_UP);
        rc = launch_pf(k_pf_swiglu, pf_lds_bytes<1, PF_BM_WIDE>(), pg, s, pf_task(tg, pg, ws, W, T, g, 0), act);
    }
    if (rc) return rc;

    if ((rc = pf_stage(1, act, F, T, F, nullptr, 0.f, ws, W, 0, 0, hd, 0.0, false, s))) return rc;
    const GemvTask td = make_task(KIND_ADJ, &L->wd, nullptr, nullptr, hd);
    const PfPlan pd = pf_plan(td.total_pairs, F, T, true, PF_BM_ROWS);
    TimeScope ts(I4D_TIME_DOWN);
    return pf_rows(pf_task(td, pd, ws, W, T, g, D), pd, x_out, y, s);
}

// One layer as phase launches (q/k/v, attention, Wo, gate/up, down), using
// the workspace region R.
int run_layer_phases(const i4d_config* c, const i4d_layer* L, int B, const float* x_in, float* x_out, const i4d_kv* kv,
                     const int* pos, int max_pos, char* ws, const WsLayout& W, char* R, hipStream_t s, int kvb) {
    const int nb = nb_slot(B), nwg = num_cus() * WG_PER_CU;
    const int hd = c->head_dim;
    int* status = (int*)(ws + WS_STATUS);
    uint16_t* kvn = (uint16_t*)(R + W.kvn);
    float* q = (float*)(R + W.q);
    float* o = (float*)(R + W.o);
    float* y = (float*)(R + W.y);
    float* act = (float*)(R + W.act);
    int rc;

    GemvTask tq = make_task(KIND_QKV, &L->wq, &L->wk, &L->wv, hd);
    const int fq = pick_fmt(L->wq, L->wk, &L->wv);
    plan_passes(tq, fq, nb, nwg, 0, GEMV_NT, 36);
    {
        TimeScope ts(I4D_TIME_QKV);
        rc = launch_qkv(fq, nb, tq, nwg, x_in, B, L->attn_norm, c->rms_eps, pos, max_pos, q, kv, kvn, c->n_q_heads,
                        c->n_kv_heads, c->rope_base, status, kvb, s);
    }
    if (rc) return rc;
    {
        TimeScope ts(I4D_TIME_ATTENTION);
        rc = launch_attention(attn_args(c, B, q, kv, kvn, pos, max_pos, o, ws, W, R, kvb), hd, s);
    }
    if (rc) return rc;

    GemvTask to = make_task(KIND_ADJ, &L->wo, nullptr, nullptr, hd);
    const int fo = pick_fmt(L->wo);
    {
        TimeScope ts(I4D_TIME_WO);
        rc = launch_rows_chunked(fo, nb, to, nwg, o, c->n_q_heads * hd, B, y, x_in, 40, s);
    }
    if (rc) return rc;

    GemvTask tg = make_task(KIND_TWO, &L->wg, &L->wu, nullptr, hd);
    const int fg = pick_fmt(L->wg, L->wu);
    plan_passes(tg, fg, nb, nwg, 0, GEMV_NT, 36);
    {
        TimeScope ts(I4D_TIME_GATE_UP);
        rc = launch_swiglu(fg, nb, tg, nwg, y, B, L->ffn_norm, c->rms_eps, act, s);
    }
    if (rc) return rc;

    GemvTask td = make_task(KIND_ADJ, &L->wd, nullptr, nullptr, hd);
    const int fd = pick_fmt(L->wd);
    TimeScope ts(I4D_TIME_DOWN);
    return launch_rows_chunked(fd, nb, td, nwg, act, c->d_ff, B, x_out, y, 40, s);
}

}  // namespace

// ============================================================== C ABI
extern "C" {

size_t i4d_workspace_size(const i4d_config* cfg, int32_t n_layers, int32_t batch, int32_t max_pos, int32_t vocab) {
    if (validate_cfg(cfg) || n_layers < 1 || batch < 1 || batch > MAX_BATCH_ALL || max_pos < 0 || vocab < 0) return 0;
    if (batch * cfg->n_kv_heads > WS_MAX_CNT) return 0;
    size_t total = ws_layout(cfg, n_layers, batch).total;
    if (batch > MAX_BATCH && vocab > 0)
        total = std::max(total, WS_LM_END + mfma_scratch(cfg->d_model, nb_mfma(batch), 0, 64).total);
    return total;
}

int i4d_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws) return I4D_EWORKSPACE;
    if (!aligned(ws, 256)) return I4D_EALIGN;
    if (ws_bytes < WS_HEADER) return I4D_EWORKSPACE;
    // the status word lives in the header; zero the whole workspace
    if (const int rc_ = scratch_free(k_fill_zero)) return rc_;
    hipLaunchKernelGGL(k_fill_zero, dim3(256), dim3(256), 0, (hipStream_t)stream, (int*)ws, ws_bytes / 4);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

int i4d_decode_layer(const i4d_config* cfg, const i4d_layer* layer, int32_t batch, const float* x_in, float* x_out,
                     const i4d_kv* kv, const int32_t* pos, int32_t max_pos, void* ws, size_t ws_bytes, void* stream) {
    return i4d_decode_stack(cfg, 1, layer, batch, x_in, x_out, kv, pos, max_pos, ws, ws_bytes, stream);
}

// run = false: validate only (nothing is enqueued)
// kvb = 1: sequence b uses its own cache (decode); 0: the batch is a chunk of
// one sequence's tokens sharing cache 0 (prefill)
static int decode_stack_impl(bool run, const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, int32_t batch,
                             const float* x_in, float* x_out, const i4d_kv* kv, const int32_t* pos, int32_t max_pos,
                             void* ws, size_t ws_bytes, void* stream, int kvb = 1) {
    int rc;
    if ((rc = validate_cfg(cfg))) return rc;
    if (n_layers < 1 || !layers || !kv) return I4D_EINVAL;
    if (batch < 1 || batch > MAX_BATCH_ALL) return I4D_ERANGE;
    if (!x_in || !x_out || !pos || x_in == x_out) return I4D_EINVAL;
    if (!aligned(x_in, 16) || !aligned(x_out, 16) || !aligned(pos, 4)) return I4D_EALIGN;
    if (cfg->d_model % 8 != 0 || cfg->d_ff % 8 != 0) return I4D_EINVAL;
    for (int l = 0; l < n_layers; ++l) {
        if ((rc = validate_layer(cfg, &layers[l]))) return rc;
        if (layers[l].wq.dtype != layers[0].wq.dtype) return I4D_EINVAL;
        if ((rc = validate_kv(cfg, &kv[l], max_pos))) return rc;
        if (batch > MAX_BATCH) {
            if (!mfma_layer_ok(cfg, &layers[l])) return I4D_EUNSUPPORTED;
        } else if (cfg->exec_mode != 2 && phases_fit(&layers[l], batch) != I4D_OK) {
            // 5..8 sequences whose staged activations overflow LDS: the batched path
            if (batch <= MAX_BATCH / 2 || !mfma_layer_ok(cfg, &layers[l])) return I4D_EUNSUPPORTED;
        }
    }
    if (batch * cfg->n_kv_heads > WS_MAX_CNT) return I4D_EUNSUPPORTED;
    const WsLayout W = ws_layout(cfg, n_layers, batch);
    if ((rc = validate_ws(ws, ws_bytes, W.total))) return rc;
    char* w = (char*)ws;
    hipStream_t s = (hipStream_t)stream;
    // the streaming kernel: exec_mode 2, or auto when the request qualifies
    const bool stream_ok = kvb == 1 && W.stream != 0 && i4d_stream::supported(cfg, n_layers, layers, kv, batch, num_cus());
    if (cfg->exec_mode == 2 && !stream_ok) return I4D_EUNSUPPORTED;
    if (stream_ok && cfg->exec_mode != 1) {
        if (!run) return I4D_OK;
        TimeScope ts(I4D_TIME_STREAM);
        const int slot = take_timing_slot();
        return i4d_stream::run(cfg, n_layers, layers, x_in, x_out, kv, pos, max_pos, w + W.stream, (int*)(w + WS_STATUS),
                               (unsigned*)(w + WS_EPOCH), num_cus(), s, slot >= 0 ? &g_timing.ev[2 * slot] : nullptr);
    }
    if (!run) return I4D_OK;
    for (int l = 0; l < n_layers; ++l) {
        char* R = w + W.layer0 + (size_t)l * W.layer_stride;
        const float* in = (l == 0) ? x_in : (const float*)(R - W.layer_stride + W.x);
        float* out = (l == n_layers - 1) ? x_out : (float*)(R + W.x);
        const bool batched = batch > MAX_BATCH || phases_fit(&layers[l], batch) != I4D_OK;
        rc = batched ? run_layer_mfma(cfg, &layers[l], batch, in, out, &kv[l], pos, max_pos, w, W, R, s, kvb)
                     : run_layer_phases(cfg, &layers[l], batch, in, out, &kv[l], pos, max_pos, w, W, R, s, kvb);
        if (rc) return rc;
    }
    return I4D_OK;
}

int i4d_decode_stack(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, int32_t batch, const float* x_in,
                     float* x_out, const i4d_kv* kv, const int32_t* pos, int32_t max_pos, void* ws, size_t ws_bytes,
                     void* stream) {
    return decode_stack_impl(true, cfg, n_layers, layers, batch, x_in, x_out, kv, pos, max_pos, ws, ws_bytes, stream);
}

// run = false: validate only (nothing is enqueued)
static int lm_head_impl(bool run, const i4d_mat* w_lm, int32_t batch, const float* h, int32_t chunk_rows, int32_t* token_out,
                        float* max_logit_out, void* ws, size_t ws_bytes, void* stream,
                        const Sampler& smp = Sampler{0.f, 0u, 0u, nullptr}) {
    if (!w_lm || w_lm->dtype != I4D_WEIGHT_INT4) return I4D_EINVAL;
    int rc;
    if ((rc = validate_mat(w_lm, w_lm->n, w_lm->k, I4D_WEIGHT_INT4, w_lm->group))) return rc;
    if (w_lm->n < 1 || w_lm->k < 8) return I4D_EINVAL;
    if (batch < 1 || batch > MAX_BATCH_ALL || chunk_rows <= 0) return I4D_ERANGE;
    if (!h || !token_out || !max_logit_out) return I4D_EINVAL;
    if (!aligned(h, 16)) return I4D_EALIGN;
    if ((rc = validate_ws(ws, ws_bytes, WS_LM_KEYS + WS_LM_BYTES))) return rc;
    char* w = (char*)ws;
    hipStream_t s = (hipStream_t)stream;
    if (batch > MAX_BATCH) {
        // batched: staging + MFMA GEMM with per-lane argmax keys (the K axis is not split)
        if (!mfma_mat_ok(*w_lm)) return I4D_EUNSUPPORTED;
        const int nb = nb_mfma(batch);
        const MfmaScratch S = mfma_scratch(w_lm->k, nb, 0, 64);
        if ((rc = validate_ws(ws, ws_bytes, WS_LM_END + S.total))) return rc;
        const GemvTask t = make_task(KIND_ADJ, w_lm, nullptr, nullptr, 64);
        const MfmaPlan p = mfma_plan(t.total_pairs, w_lm->k, nb, 1, false);
        if (p.nwg > LM_MAX_WG) return I4D_EUNSUPPORTED;
        if (!run) return I4D_OK;
        if ((rc = scratch_free(k_lm_finalize))) return rc;
        char* base = w + WS_LM_END;
        if ((rc = mfma_stage(1, nb, h, w_lm->k, batch, w_lm->k, nullptr, 0.f, base, S, nullptr, 0, 0, 64, 0.0, false,
                             (int*)(w + WS_STATUS), s)))
            return rc;
        const MfmaTask m = mfma_task(t, p, base, S, nullptr, batch, w_lm->group);
        u64* keys = (u64*)(w + WS_LM_KEYS);
        {
            TimeScope ts(I4D_TIME_LM_HEAD);
            rc = nb == 16 ? launch_mfma(k_mfma_lm<16>, MfmaGeo<16, 1>::LDS_B, p, s, m, keys, smp)
                          : launch_mfma(k_mfma_lm<32>, MfmaGeo<32, 1>::LDS_B, p, s, m, keys, smp);
        }
        if (rc) return rc;
        hipLaunchKernelGGL(k_lm_finalize, dim3(1), dim3(256), 0, s, (const u64*)keys, p.nwg, nb, batch, token_out, max_logit_out);
        return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
    }
    const int nb = nb_slot(batch), nwg = num_cus() * WG_PER_CU;
    GemvTask t = make_task(KIND_ADJ, w_lm, nullptr, nullptr, 64);
    const int fmt = pick_fmt(*w_lm);
    // Logits only ever exist in registers (each workgroup keeps a running
    // maximum), so nothing is gained by passes as small as chunk_rows: the
    // passes are as large as the per-workgroup run budget allows.
    plan_passes(t, fmt, nb, nwg, 0, GEMV_NT, 34);
    if (nwg > LM_MAX_WG) return I4D_EUNSUPPORTED;
    if (!run) return I4D_OK;
    TimeScope ts(I4D_TIME_LM_HEAD);
    return launch_lm(fmt, nb, t, nwg, h, batch, (u64*)(w + WS_LM_KEYS), token_out, max_logit_out, smp, s);
}

// ---- greedy LM head without a workspace
// The matrix-vector LM head's only scratch is the per-workgroup argmax keys
// (every workgroup writes its own before the finalising kernel reads them, so
// nothing needs clearing).  This variant keeps them in a file-scope device
// array instead of the caller's workspace.  Host code must not pass the
// array's name to a kernel: the name is a host-side stand-in; the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current (each GPU holds its own copy of the array).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)LM_MAX_WG * MAX_BATCH * sizeof(u64);   // 256 KiB
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static int scratch_device_ptr(u64** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return I4D_EHIP;
    static std::mutex mu;
    static void* ptrs[NOALLOC_MAX_DEVICES] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return I4D_EHIP;
        ptrs[dev] = ptr;
    }
    *out = (u64*)ptrs[dev];
    return I4D_OK;
}

int i4d_lm_head_chunked_noalloc(const i4d_mat* w_lm, int32_t batch, const float* h, int32_t chunk_rows, int32_t* token_out,
                                float* max_logit_out, void* stream) {
    if (!w_lm || w_lm->dtype != I4D_WEIGHT_INT4) return I4D_EINVAL;
    int rc;
    if ((rc = validate_mat(w_lm, w_lm->n, w_lm->k, I4D_WEIGHT_INT4, w_lm->group))) return rc;
    if (w_lm->n < 1 || w_lm->k < 8) return I4D_EINVAL;
    if (batch < 1 || batch > MAX_BATCH || chunk_rows <= 0) return I4D_ERANGE;
    if (!h || !token_out || !max_logit_out) return I4D_EINVAL;
    if (!aligned(h, 16)) return I4D_EALIGN;
    const int nb = nb_slot(batch), nwg = num_cus() * WG_PER_CU;
    GemvTask t = make_task(KIND_ADJ, w_lm, nullptr, nullptr, 64);
    const int fmt = pick_fmt(*w_lm);
    plan_passes(t, fmt, nb, nwg, 0, GEMV_NT, 34);
    if ((size_t)nwg * MAX_BATCH * sizeof(u64) > NOALLOC_SCRATCH_BYTES) return I4D_ERANGE;
    u64* keys = nullptr;
    if ((rc = scratch_device_ptr(&keys))) return rc;
    return launch_lm(fmt, nb, t, nwg, h, batch, keys, token_out, max_logit_out, Sampler{0.f, 0u, 0u, nullptr},
                     (hipStream_t)stream);
}

// Host checks of the sampling arguments; the sampler of a valid set.
static int make_sampler(float temperature, uint64_t seed, const int32_t* counter, Sampler& smp) {
    if (!counter) return I4D_EINVAL;
    if (!aligned(counter, 4)) return I4D_EALIGN;
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return I4D_EINVAL;
    const float inv_t = (float)(1.0 / (double)temperature);
    if (!std::isfinite(inv_t) || !std::isnormal(inv_t)) return I4D_EINVAL;
    smp = Sampler{inv_t, (u32)(seed & 0xFFFFFFFFu), (u32)(seed >> 32), counter};
    return I4D_OK;
}

int i4d_lm_head_chunked(const i4d_mat* w_lm, int32_t batch, const float* h, int32_t chunk_rows, int32_t* token_out,
                        float* max_logit_out, void* ws, size_t ws_bytes, void* stream) {
    return lm_head_impl(true, w_lm, batch, h, chunk_rows, token_out, max_logit_out, ws, ws_bytes, stream);
}

int i4d_lm_head_sample(const i4d_mat* w_lm, int32_t batch, const float* h, int32_t chunk_rows, float temperature,
                       uint64_t seed, const int32_t* counter, int32_t* token_out, float* score_out, void* ws, size_t ws_bytes,
                       void* stream) {
    Sampler smp;
    int rc;
    if ((rc = make_sampler(temperature, seed, counter, smp))) return rc;
    return lm_head_impl(true, w_lm, batch, h, chunk_rows, token_out, score_out, ws, ws_bytes, stream, smp);
}

int i4d_prefill_chunk(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, int32_t n_tokens, const float* x_in,
                      float* x_out, const i4d_kv* kv, const int32_t* pos, int32_t max_pos, void* ws, size_t ws_bytes,
                      void* stream) {
    return decode_stack_impl(true, cfg, n_layers, layers, n_tokens, x_in, x_out, kv, pos, max_pos, ws, ws_bytes, stream, 0);
}

size_t i4d_prefill_workspace_size(const i4d_config* cfg, int32_t n_tokens) {
    if (validate_cfg(cfg) || n_tokens < 1 || n_tokens > I4D_PREFILL_MAX_TOKENS) return 0;
    return pf_ws(cfg, n_tokens).total;
}

int i4d_prefill(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, int32_t n_tokens, const float* x_in,
                float* x_out, const i4d_kv* kv, int32_t pos0, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = validate_cfg(cfg))) return rc;
    if (n_layers < 1 || !layers || !kv || !x_in || !x_out) return I4D_EINVAL;
    if (n_tokens < 1 || n_tokens > I4D_PREFILL_MAX_TOKENS || pos0 < 0) return I4D_ERANGE;
    if (!aligned(x_in, 16) || !aligned(x_out, 16)) return I4D_EALIGN;
    const PfWs W = pf_ws(cfg, n_tokens);
    if ((rc = validate_ws(ws, ws_bytes, W.total))) return rc;
    const long long last = (long long)pos0 + n_tokens - 1;
    if (last > INT32_MAX) return I4D_ERANGE;
    for (int l = 0; l < n_layers; ++l) {
        if ((rc = validate_layer(cfg, &layers[l]))) return rc;
        if ((rc = validate_kv(cfg, &kv[l], (int)last))) return rc;
        if (layers[l].wq.dtype != I4D_WEIGHT_INT4 || !mfma_layer_ok(cfg, &layers[l])) return I4D_EUNSUPPORTED;
        if (layers[l].wq.group != layers[0].wq.group) return I4D_EUNSUPPORTED;
    }
    char* w = (char*)ws;
    hipStream_t s = (hipStream_t)stream;
    if ((rc = scratch_free(k_pf_positions))) return rc;
    hipLaunchKernelGGL(k_pf_positions, dim3((n_tokens + 255) / 256), dim3(256), 0, s, (int*)(w + W.pos), n_tokens, pos0);
    if (hipGetLastError() != hipSuccess) return I4D_EHIP;
    const float* in = x_in;
    for (int l = 0; l < n_layers; ++l) {
        float* out = (l == n_layers - 1) ? x_out : (float*)(w + ((l & 1) ? W.xb : W.xa));
        if ((rc = run_layer_prefill(cfg, &layers[l], n_tokens, in, out, &kv[l], pos0, w, W, s))) return rc;
        in = out;
    }
    return I4D_OK;
}

int i4d_embed(const uint16_t* table, int32_t vocab, int32_t d_model, int32_t batch, const int32_t* tokens, float* x_out,
              void* ws, size_t ws_bytes, void* stream) {
    if (!table || !tokens || !x_out || !ws) return I4D_EINVAL;
    if (vocab < 1 || d_model < 1) return I4D_EINVAL;
    if (batch < 1 || batch > MAX_BATCH_ALL) return I4D_ERANGE;
    if (!aligned(table, 2) || !aligned(tokens, 4) || !aligned(x_out, 4)) return I4D_EALIGN;
    int rc;
    if ((rc = validate_ws(ws, ws_bytes, WS_HEADER))) return rc;
    const dim3 grid((d_model + 255) / 256, batch);
    if (const int rc_ = scratch_free(k_embed)) return rc_;
    hipLaunchKernelGGL(k_embed, grid, dim3(256), 0, (hipStream_t)stream, table, vocab, d_model, tokens, x_out,
                       (int*)((char*)ws + WS_STATUS));
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

// Workspace of top-k sampling: the LM head GEMV's own scratch (batches above
// 8), then the logits [B][V] fp32 and the slices' candidate keys [B][slices][k].
struct TopkWs { size_t logits, cand, total; int slices; };
static int topk_ws(const i4d_mat* w_lm, int batch, int top_k, TopkWs& t) {
    size_t off = WS_HEADER;
    if (batch > MAX_BATCH) {
        if (!mfma_mat_ok(*w_lm)) return I4D_EUNSUPPORTED;
        const int nb = nb_mfma(batch);
        const GemvTask tk = make_task(KIND_ADJ, w_lm, nullptr, nullptr, 64);
        const MfmaPlan p = mfma_plan(tk.total_pairs, w_lm->k, nb, 1, true);
        off = WS_LM_END + mfma_scratch(w_lm->k, nb, mfma_part_bytes(p, nb), 64).total;
    }
    t.slices = (w_lm->n + TOPK_SLICE - 1) / TOPK_SLICE;
    if ((long long)t.slices * top_k > TOPK_MERGE_MAX) return I4D_EUNSUPPORTED;
    t.logits = align256(off);
    t.cand = align256(t.logits + (size_t)batch * w_lm->n * 4);
    t.total = t.cand + (size_t)batch * t.slices * top_k * 8;
    return I4D_OK;
}

static int lm_head_topk_impl(bool run, const i4d_mat* w_lm, int32_t batch, const float* h, int32_t top_k, float temperature,
                             uint64_t seed, const int32_t* counter, int32_t* token_out, float* score_out, void* ws,
                             size_t ws_bytes, void* stream) {
    if (!w_lm || w_lm->dtype != I4D_WEIGHT_INT4) return I4D_EINVAL;
    int rc;
    if ((rc = validate_mat(w_lm, w_lm->n, w_lm->k, I4D_WEIGHT_INT4, w_lm->group))) return rc;
    if (w_lm->n < 1 || w_lm->k < 8) return I4D_EINVAL;
    if (batch < 1 || batch > MAX_BATCH_ALL) return I4D_ERANGE;
    if (top_k < 1 || top_k > TOPK_MAX || top_k > w_lm->n) return I4D_ERANGE;
    if (!h || !token_out || !score_out || !counter) return I4D_EINVAL;
    if (!aligned(h, 16) || !aligned(counter, 4)) return I4D_EALIGN;
    Sampler smp;
    if ((rc = make_sampler(temperature, seed, counter, smp))) return rc;
    TopkWs T;
    if ((rc = topk_ws(w_lm, batch, top_k, T))) return rc;
    if ((rc = validate_ws(ws, ws_bytes, T.total))) return rc;
    if (!run) return I4D_OK;
    char* w = (char*)ws;
    float* logits = (float*)(w + T.logits);
    u64* cand = (u64*)(w + T.cand);
    hipStream_t s = (hipStream_t)stream;
    {
        TimeScope ts(I4D_TIME_LM_HEAD);
        if ((rc = i4d_gemv(w_lm, batch, h, logits, ws, ws_bytes, stream))) return rc;
    }
    if ((rc = scratch_free(k_topk_slice)) || (rc = scratch_free(k_topk_sample))) return rc;
    hipLaunchKernelGGL(k_topk_slice, dim3(T.slices, batch), dim3(512), 0, s, (const float*)logits, w_lm->n, top_k, cand);
    if (hipGetLastError() != hipSuccess) return I4D_EHIP;
    const int n = T.slices * top_k;
    int np2 = 1;
    while (np2 < n) np2 <<= 1;
    if ((rc = set_lds(k_topk_sample, (size_t)np2 * 8))) return rc;
    hipLaunchKernelGGL(k_topk_sample, dim3(batch), dim3(1024), (size_t)np2 * 8, s, (const u64*)cand, n, np2, top_k, smp,
                       token_out, score_out);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

size_t i4d_topk_workspace_size(const i4d_mat* w_lm, int32_t batch, int32_t top_k) {
    if (!w_lm || w_lm->n < 1 || batch < 1 || batch > MAX_BATCH_ALL || top_k < 1 || top_k > TOPK_MAX) return 0;
    TopkWs T;
    if (topk_ws(w_lm, batch, top_k, T)) return 0;
    return T.total;
}

int i4d_lm_head_sample_topk(const i4d_mat* w_lm, int32_t batch, const float* h, int32_t top_k, float temperature,
                            uint64_t seed, const int32_t* counter, int32_t* token_out, float* score_out, void* ws,
                            size_t ws_bytes, void* stream) {
    return lm_head_topk_impl(true, w_lm, batch, h, top_k, temperature, seed, counter, token_out, score_out, ws, ws_bytes,
                             stream);
}

// top_k > 0: the token is drawn by top-k sampling at (temperature, seed)
static int decode_step_impl(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, const uint16_t* embed,
                            const i4d_mat* w_lm, int32_t batch, int32_t* tokens, float* max_logit_out, int32_t* pos,
                            int32_t max_pos, float* x_buf, const i4d_kv* kv, void* ws, size_t ws_bytes, void* stream,
                            const Sampler& smp, int top_k = 0, float temperature = 0.f, uint64_t seed = 0) {
    int rc;
    if ((rc = validate_cfg(cfg))) return rc;
    if (!embed || !w_lm || !tokens || !pos || !x_buf) return I4D_EINVAL;
    if (!aligned(embed, 2) || !aligned(tokens, 4)) return I4D_EALIGN;
    if (w_lm->k != cfg->d_model) return I4D_EINVAL;
    const size_t plane = (size_t)batch * cfg->d_model;
    float* x0 = x_buf;
    float* x1 = x_buf + plane;
    // every check before anything is enqueued
    if ((rc = decode_stack_impl(false, cfg, n_layers, layers, batch, x0, x1, kv, pos, max_pos, ws, ws_bytes, stream))) return rc;
    auto head = [&](bool run) {
        return top_k > 0 ? lm_head_topk_impl(run, w_lm, batch, x1, top_k, temperature, seed, pos, tokens, max_logit_out, ws,
                                             ws_bytes, stream)
                         : lm_head_impl(run, w_lm, batch, x1, 8192, tokens, max_logit_out, ws, ws_bytes, stream, smp);
    };
    if ((rc = head(false))) return rc;
    if (top_k > 0) {
        // the sampling scratch must not reach the streaming kernel's region,
        // whose exchange words carry over from step to step
        TopkWs T;
        if ((rc = topk_ws(w_lm, batch, top_k, T))) return rc;
        const WsLayout W = ws_layout(cfg, n_layers, batch);
        if (W.stream != 0 && T.total > W.stream) return I4D_EUNSUPPORTED;
    }
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((cfg->d_model + 255) / 256, batch);
    if (const int rc_ = scratch_free(k_embed)) return rc_;
    if (const int rc_ = scratch_free(k_advance)) return rc_;
    hipLaunchKernelGGL(k_embed, grid, dim3(256), 0, s, embed, w_lm->n, cfg->d_model, (const int*)tokens, x0,
                       (int*)((char*)ws + WS_STATUS));
    if (hipGetLastError() != hipSuccess) return I4D_EHIP;
    if ((rc = decode_stack_impl(true, cfg, n_layers, layers, batch, x0, x1, kv, pos, max_pos, ws, ws_bytes, stream))) return rc;
    if ((rc = head(true))) return rc;
    hipLaunchKernelGGL(k_advance, dim3(1), dim3(64), 0, s, pos, batch);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

int i4d_decode_step(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, const uint16_t* embed,
                    const i4d_mat* w_lm, int32_t batch, int32_t* tokens, float* max_logit_out, int32_t* pos,
                    int32_t max_pos, float* x_buf, const i4d_kv* kv, void* ws, size_t ws_bytes, void* stream) {
    return decode_step_impl(cfg, n_layers, layers, embed, w_lm, batch, tokens, max_logit_out, pos, max_pos, x_buf, kv, ws,
                            ws_bytes, stream, Sampler{0.f, 0u, 0u, nullptr});
}

int i4d_decode_step_sample(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, const uint16_t* embed,
                           const i4d_mat* w_lm, int32_t batch, int32_t* tokens, float* score_out, int32_t* pos,
                           int32_t max_pos, float* x_buf, const i4d_kv* kv, float temperature, uint64_t seed, void* ws,
                           size_t ws_bytes, void* stream) {
    Sampler smp;
    int rc;
    // the counter word of sequence b is its position pos[b] (read before the advance)
    if ((rc = make_sampler(temperature, seed, pos, smp))) return rc;
    return decode_step_impl(cfg, n_layers, layers, embed, w_lm, batch, tokens, score_out, pos, max_pos, x_buf, kv, ws,
                            ws_bytes, stream, smp);
}

int i4d_decode_step_sample_topk(const i4d_config* cfg, int32_t n_layers, const i4d_layer* layers, const uint16_t* embed,
                                const i4d_mat* w_lm, int32_t batch, int32_t* tokens, float* score_out, int32_t* pos,
                                int32_t max_pos, float* x_buf, const i4d_kv* kv, int32_t top_k, float temperature,
                                uint64_t seed, void* ws, size_t ws_bytes, void* stream) {
    if (top_k < 1) return I4D_ERANGE;
    // the counter word of sequence b is its position pos[b] (read before the advance)
    return decode_step_impl(cfg, n_layers, layers, embed, w_lm, batch, tokens, score_out, pos, max_pos, x_buf, kv, ws,
                            ws_bytes, stream, Sampler{0.f, 0u, 0u, nullptr}, top_k, temperature, seed);
}

int i4d_dequant_int4(const i4d_mat* wm, float* out, void* stream) {
    if (!wm || !out) return I4D_EINVAL;
    int rc;
    if ((rc = validate_mat(wm, wm->n, wm->k, I4D_WEIGHT_INT4, wm->group))) return rc;
    const int ng = (wm->k + wm->group - 1) / wm->group;
    if (const int rc_ = scratch_free(k_dequant)) return rc_;
    hipLaunchKernelGGL(k_dequant, dim3(1024), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)wm->data,
                       (const uint16_t*)wm->scales, wm->n, wm->k, wm->group, ng, out);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

int i4d_gemv(const i4d_mat* wm, int32_t batch, const float* x, float* y, void* ws, size_t ws_bytes, void* stream) {
    if (!wm || !x || !y) return I4D_EINVAL;
    int rc;
    if ((rc = validate_mat(wm, wm->n, wm->k, wm->dtype, wm->group))) return rc;
    if (wm->n < 1) return I4D_EINVAL;
    if (batch < 1 || batch > MAX_BATCH_ALL) return I4D_ERANGE;
    if (!aligned(x, 16) || !aligned(y, 4)) return I4D_EALIGN;
    if (batch > MAX_BATCH) {
        // batched: staging + MFMA GEMM; scratch after the workspace's LM-head keys
        if (!mfma_mat_ok(*wm)) return I4D_EUNSUPPORTED;
        const int nb = nb_mfma(batch);
        const GemvTask t = make_task(KIND_ADJ, wm, nullptr, nullptr, 64);
        const MfmaPlan p = mfma_plan(t.total_pairs, wm->k, nb, 1, true);
        const MfmaScratch S = mfma_scratch(wm->k, nb, mfma_part_bytes(p, nb), 64);
        if ((rc = validate_ws(ws, ws_bytes, WS_LM_END + S.total))) return rc;
        char* w = (char*)ws;
        char* base = w + WS_LM_END;
        hipStream_t s = (hipStream_t)stream;
        if ((rc = mfma_stage(1, nb, x, wm->k, batch, wm->k, nullptr, 0.f, base, S, nullptr, 0, 0, 64, 0.0, false,
                             (int*)(w + WS_STATUS), s)))
            return rc;
        return mfma_rows(nb, mfma_task(t, p, base, S, (int*)(w + WS_MCNT), batch, wm->group), p, y, nullptr, s);
    }
    const int nb = nb_slot(batch), nwg = num_cus() * WG_PER_CU;
    GemvTask t = make_task(KIND_ADJ, wm, nullptr, nullptr, 64);
    const int fmt = pick_fmt(*wm);
    plan_passes(t, fmt, nb, nwg, 0, GEMV_NT, 36);
    return launch_rows(fmt, nb, t, nwg, x, wm->k, batch, nullptr, 0.f, y, nullptr, (hipStream_t)stream);
}

int i4d_attention(const i4d_config* cfg, int32_t batch, const float* q, const i4d_kv* kv, const int32_t* pos, int32_t max_pos,
                  float* o, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = validate_cfg(cfg))) return rc;
    if (batch < 1 || batch > MAX_BATCH_ALL) return I4D_ERANGE;
    if (!q || !o || !pos) return I4D_EINVAL;
    if ((rc = validate_kv(cfg, kv, max_pos))) return rc;
    const WsLayout W = ws_layout(cfg, 1, batch);
    if ((rc = validate_ws(ws, ws_bytes, W.total))) return rc;
    if (batch * cfg->n_kv_heads > WS_MAX_CNT) return I4D_EUNSUPPORTED;
    char* w = (char*)ws;
    return launch_attention(attn_args(cfg, batch, q, kv, nullptr, pos, max_pos, o, w, W, w + W.layer0), cfg->head_dim,
                            (hipStream_t)stream);
}

int i4d_launch_timing_start(int32_t kernel, int32_t max_launches) {
    if (kernel < I4D_TIME_QKV || kernel > I4D_TIME_STREAM || max_launches < 1 || max_launches > 65536)
        return I4D_EINVAL;
    g_timing.kind = 0;
    g_timing.n = 0;
    while ((int)g_timing.ev.size() < 2 * max_launches) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return I4D_EHIP;
        g_timing.ev.push_back(e);
    }
    g_timing.cap = max_launches;
    g_timing.kind = kernel;
    return I4D_OK;
}

int i4d_launch_timing_stop(float* total_ms, int32_t* launches) {
    if (!total_ms || !launches) return I4D_EINVAL;
    const int n = g_timing.n;
    g_timing.kind = 0;
    g_timing.n = 0;
    *total_ms = 0.f;
    *launches = n;
    if (n == 0) return I4D_OK;
    double sum = 0.0;
    for (int i = 0; i < n; ++i) {                  // launches may have gone to several streams
        float ms = 0.f;
        if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess) return I4D_EHIP;
        if (hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess) return I4D_EHIP;
        sum += ms;
    }
    *total_ms = (float)sum;
    return I4D_OK;
}

int i4d_read_device_status(const void* ws, int32_t* status_out, void* stream) {
    if (!ws || !status_out) return I4D_EINVAL;
    if (hipMemcpyAsync(status_out, ws, sizeof(int32_t), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess) return I4D_EHIP;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return I4D_EHIP;
    return I4D_OK;
}

int i4d_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes == 0) return I4D_EINVAL;
    if (!aligned(buf, 16) || bytes % 16 || !aligned(sink, 4)) return I4D_EALIGN;
    if (const int rc_ = scratch_free(k_read_probe)) return rc_;
    hipLaunchKernelGGL(k_read_probe, dim3(num_cus()), dim3(512), 0, (hipStream_t)stream, (const u32x4*)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? I4D_OK : I4D_EHIP;
}

const char* i4d_status_string(int status) {
    switch (status) {
        case I4D_OK: return "ok";
        case I4D_EINVAL: return "invalid argument (null pointer, shape, group or head layout)";
        case I4D_EALIGN: return "misaligned pointer";
        case I4D_EWORKSPACE: return "workspace missing or too small";
        case I4D_ERANGE: return "value out of range (batch, max_pos or chunk_rows)";
        case I4D_EHIP: return "HIP launch failed";
        case I4D_EUNSUPPORTED: return "request not supported by this build";
        default: return "unknown status";
    }
}

}  // extern "C"
