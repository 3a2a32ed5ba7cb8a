// Batched int4 dequant-GEMM on the matrix cores, for 9..32 sequences per step
// (gfx950, wave64, v_mfma_f32_16x16x32_f16).
//
// At batch 16 and above every weight byte feeds 16-32 multiply-adds, beyond
// what the vector ALUs sustain at HBM speed (the roofline reply, 二 and 三:
// batching raises arithmetic intensity; the Unsloth article, 二.3: int4
// codes are expanded in registers).  The weights stay a stream read once per
// step; only the dot products move to MFMA.
//
// Operands of one 16x16x32 MFMA (C[m][n] += sum_k A[m][k] B[k][n]):
//   A = activations: m = sequence (16 per N-tile), 8 halves per lane;
//   B = weights:     n = output row of a 16-row tile, 8 halves per lane;
//   C: lane (r = lane & 15, q = lane >> 4) receives C[4q + e][r], e = 0..3,
//      i.e. four sequences of output row r.
// A and B pair their register elements by the same (lane group, element)
// index, so the order of the K axis inside one instruction is free: it is the
// order the int4 unpack produces, and the staged activations follow it.
//
// Row tile.  A tile is 8 consecutive pairs of the task (gate/up row i with
// up row i, RoPE pair (i, i + hd/2), or two adjacent rows): lane r < 8
// streams row a of pair 8t + r, lane r >= 8 row b of pair 8t + r - 8, so an
// epilogue finds the two rows of a pair in lanes r and r ^ 8.
//
// Step.  One step covers 128 inputs of every row of a tile: lane group q
// takes the 16 bytes (32 inputs) at byte 64 s + 16 q of its row, and dword j
// of them is the B operand of MFMA j (j = 0..3).  The bytes are loaded two
// steps at a time as whole 128-byte lines (eight rows per load instruction)
// and rearranged through LDS; the scales of a chunk's groups are loaded once
// per chunk and passed between lanes.  With groups of 128
// inputs (or a power-of-two multiple) a step lies inside one group, so the
// four MFMAs of a step accumulate into a fresh tile that is then scaled by
// the lane's own row scale and added to the running sum:
//   sum_k (c_k - 8) s x_k = s * C_step.
// The unpack makes exact fp16 weights: OR-ing the masked nibbles into fp16
// 1024 gives 1024 + c (even inputs) and 1024 + 16 c (odd inputs), and one
// packed subtract of 1032 or 1152 leaves c - 8 and 16 (c - 8); the staged odd
// activations are pre-divided by 16 (exact).  The MFMA then sums products of
// the true magnitudes, so its fp32 accumulation carries no large bias.
//
// Work split.  A workgroup (8 waves) owns a row block of 8*RT tiles and one
// block of the K axis; each wave streams RT tiles over that K block.  The
// K block's staged activations pass through LDS in chunks of SC steps
// (double-buffered; the next chunk is loaded into registers while the
// current one is consumed).  When the K axis is split over several
// workgroups, each writes its partial sums through to memory and the last of
// them to arrive (an arrival counter per row block) adds the K blocks in
// block order and runs the epilogue, so results do not depend on timing.
#pragma once
#include "common.h"
#include "gemv.h"

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

template <int NB, int PREC>
struct MfmaGeo {
    static constexpr int NT = 512;                                   // threads per workgroup
    static constexpr int NTL = NB / 16;                              // 16-sequence N-tiles
    static constexpr int RT = (NB == 32 && PREC == 1) ? 2 : 1;       // row tiles per wave
    static constexpr int TB = 8 * RT;                                // row tiles per workgroup
    static constexpr int SC = 4;                                     // steps per LDS chunk
    static constexpr int D = 2;                                      // step pairs of weight loads in flight
    static constexpr int ROW_B = SC * 256 + 16;                      // LDS pitch of one staged row (padded)
    static constexpr int ACT_B = PREC * NB * ROW_B;                  // one chunk buffer
    static constexpr int CHUNK_LOADS = PREC * NB * SC * 16;          // 16-byte pieces per chunk
    static constexpr int LPT = (CHUNK_LOADS + NT - 1) / NT;          // pieces per thread
    static constexpr int WROW_B = 144;                               // one tile row of a step pair in LDS (padded)
    static constexpr int WT_B = 16 * WROW_B;                         // one tile's step pair
    static constexpr int WAVE_W_B = RT * WT_B;                       // a wave's weight transpose area
    static constexpr int LDS_B = 2 * ACT_B + (NT / 64) * WAVE_W_B + (NT / 64) * NB * 8 + 64;
    static_assert((SC / 2) % D == 0, "chunk length must be a multiple of the ring depth");
};

// One batched GEMM phase.
struct MfmaTask {
    GemvTask t;                // matrices and pair mapping (int4, fast layout)
    const uint32_t* xs;        // staged activations: fp16 pairs [PREC][NB][K/2] (uint32 = two halves)
    const float* xscale;       // [NB] power of two that multiplies sequence b's results (its row was staged times its inverse)
    float* part;               // partial sums [tiles][kb][NB][16] (K split only)
    int* cnt;                  // arrival counters, one per row block (K split only)
    int tiles;                 // ceil(total_pairs / 8)
    int kb;                    // K blocks
    int spb;                   // steps per K block (the last may be shorter)
    int nsteps;                // K / 128
    int gshift;                // log2(group / 128)
    int nb;                    // live sequences
};

// ---------------------------------------------------------------- staging
// One workgroup per sequence slot b < NB (slots >= nb are zero-filled).
// x is RMS-normalised with `gain` when one is given (h = x / sqrt(mean x^2 +
// eps) * gain), converted to fp16 in the unpack's order ((0,4), (1,5), (2,6),
// (3,7) of every 8 inputs, odd ones divided by 16), optionally with a second
// plane holding the fp16 of the remainder.  fp16 range: the row is staged
// times 2^-e, e = 0 unless its largest staged magnitude reaches 2^15, and
// xscale[b] = 2^e multiplies the sequence's results (both exact).
// RoPE set-up rides along for the q/k/v phase: slot b validates pos[b]
// (pos_out[b] = -1 and the status bit when out of range) and writes the
// float64-derived cos/sin of its angles, cs[b][i] for i < hd/2.
template <int PREC>
__global__ void __launch_bounds__(256) k_mfma_stage(const float* x, int x_stride, int nb, int NBP, int K, const uint16_t* gain,
                                                    float eps, uint32_t* xs,
                                                    const int* pos, int max_pos, int cap, int hd, double base,
                                                    int* pos_out, float2* cs, int* status, float* xscale) {
    __shared__ float red[4];
    __shared__ float redm[4];
    const int b = blockIdx.x, tid = i4d_tid();
    const int nsteps = K >> 7;
    const bool live = b < nb;
    const float* xb = x + (size_t)(live ? b : 0) * x_stride;

    if (pos_out != nullptr) {
        int p = -1;
        if (live) {
            p = pos[b];
            if (p < 0 || p > max_pos || p >= cap) { raise_status(status, I4D_DEV_BAD_POS); p = -1; }
        }
        if (tid == 0) pos_out[b] = p;
        const int half = hd >> 1;
        for (int i = tid; i < half; i += 256) {
            const double theta = pow(base, -2.0 * (double)i / (double)hd);
            const double phi = (double)max(p, 0) * theta;
            cs[(size_t)b * half + i] = float2{(float)cos(phi), (float)sin(phi)};
        }
    }

    float rs = 1.0f;
    if (live && gain != nullptr) {
        float ss = 0.f;
        for (int k = tid * 4; k < K; k += 1024) {
            const f4 v = ld_g((const f4*)(xb + k));
            ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
        }
        for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor_f(ss, m);
        if ((tid & 63) == 0) red[tid >> 6] = ss;
        __syncthreads();
        rs = 1.0f / sqrtf((((red[0] + red[1]) + red[2]) + red[3]) / (float)K + eps);
    }

    // the staged values of 8-input chunk c (odd ones divided by 16)
    auto staged = [&](int c, float (&a)[8]) {
        const int k0 = c * 8;
        if (live) {
            const f4 a0 = ld_g((const f4*)(xb + k0)), a1 = ld_g((const f4*)(xb + k0 + 4));
            a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w; a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
            if (gain != nullptr) {
                const u32x4 gw = ld_g((const u32x4*)(gain + k0));
                const u32 g4[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const u32 w = g4[e >> 1];
                    a[e] = a[e] * rs * __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
                }
            }
#pragma unroll
            for (int e = 1; e < 8; e += 2) a[e] *= 0.0625f;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = 0.f;
        }
    };
    // the row's power of two: largest staged |a| below 2^15 after it
    float amax = 0.f;
    for (int c = tid; c < nsteps * 16; c += 256) {
        float a[8];
        staged(c, a);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(a[e]));
    }
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, m));
    if ((tid & 63) == 0) redm[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
    int ex = 0;
    (void)frexpf(amax, &ex);                          // amax < 2^ex (0 for amax = 0)
    const int sh = max(ex - 15, 0);
    const float down = ldexpf(1.f, -sh);
    if (tid == 0) xscale[b] = ldexpf(1.f, sh);

    // 8-input chunks, one per thread per round
    for (int c = tid; c < nsteps * 16; c += 256) {
        float v[8];
        staged(c, v);
        _Float16 hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a = v[e] * down;
            hi[e] = (_Float16)a;
            lo[e] = (_Float16)(a - (float)hi[e]);
        }
        uint32_t* dst = xs + (size_t)b * (K >> 1) + (size_t)c * 4;
        u32x4 o;
        o.x = __builtin_bit_cast(u32, h2{hi[0], hi[4]});
        o.y = __builtin_bit_cast(u32, h2{hi[1], hi[5]});
        o.z = __builtin_bit_cast(u32, h2{hi[2], hi[6]});
        o.w = __builtin_bit_cast(u32, h2{hi[3], hi[7]});
        *(I4D_GLOBAL u32x4*)dst = o;
        if (PREC > 1) {
            u32x4 l;
            l.x = __builtin_bit_cast(u32, h2{lo[0], lo[4]});
            l.y = __builtin_bit_cast(u32, h2{lo[1], lo[5]});
            l.z = __builtin_bit_cast(u32, h2{lo[2], lo[6]});
            l.w = __builtin_bit_cast(u32, h2{lo[3], lo[7]});
            *(I4D_GLOBAL u32x4*)(dst + (size_t)NBP * (K >> 1)) = l;
        }
    }
}

// ---------------------------------------------------------------- the GEMM
// 8 codes of one dword -> exact fp16 (c - 8) for the even inputs and 16 (c - 8)
// for the odd ones, in the order (0,4), (1,5), (2,6), (3,7)
I4D_DEVINL h8 unpack_b(u32 w) {
    const u32 magic = 0x64006400u, w8 = w >> 8;
    const h2 ze = h2{(_Float16)-1032.0f, (_Float16)-1032.0f}, zo = h2{(_Float16)-1152.0f, (_Float16)-1152.0f};
    const h2 p0 = as_h2(and_or(w, 0x000F000Fu, magic)) + ze;
    const h2 p1 = as_h2(and_or(w, 0x00F000F0u, magic)) + zo;
    const h2 p2 = as_h2(and_or(w8, 0x000F000Fu, magic)) + ze;
    const h2 p3 = as_h2(and_or(w8, 0x00F000F0u, magic)) + zo;
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// A step pair of one tile is loaded as two fully used cache lines per row:
// instruction h (0, 1) gives lane l the 16 bytes at 16 (l & 7) of the 128-byte
// step pair of tile row 8 h + (l >> 3), i.e. eight rows of 128 bytes per
// instruction.  The wave then passes the bytes through its own LDS area into
// the MFMA layout (lane (r, q) of step s: row r, bytes 64 s + 16 q).
template <int NB, int PREC>
struct MfmaRing {
    u32x4 w[MfmaGeo<NB, PREC>::D][MfmaGeo<NB, PREC>::RT][2];
};

// Epilogue kinds of the batched path: per (pair, sequence) results go to one
// of the GEMV epilogue functors, or into per-lane argmax keys (LM head).
enum { MEPI_FN = 0, MEPI_ARGMAX = 1 };

template <int KND, int NB, int PREC, int EK, class Epi>
I4D_DEVINL void mfma_gemm(const MfmaTask& m, char* lds, Epi& epi, u64* wg_keys) {
    typedef MfmaGeo<NB, PREC> G;
    constexpr int RT = G::RT, NTL = G::NTL, SC = G::SC, D = G::D;
    const int tid = i4d_tid();
    const int wave = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
    const int rb = blockIdx.x / m.kb, kbi = blockIdx.x - rb * m.kb;
    const int s0 = kbi * m.spb, s1 = min(m.nsteps, s0 + m.spb);
    const int nst = s1 - s0;
    const int nch = (nst + SC - 1) / SC;
    const int K = m.t.k;

    char* act_buf = lds;                                         // [2][ACT_B]
    u64* key_lds = (u64*)(lds + 2 * G::ACT_B + (G::NT / 64) * G::WAVE_W_B);   // [NT/64][NB]
    int* flag = (int*)(key_lds + (G::NT / 64) * NB);

    char* wlds = lds + 2 * G::ACT_B + wave * G::WAVE_W_B;       // this wave's weight transpose area

    // rows streamed by this lane: whole-line loads (tile row 8h + lane / 8)
    // and, in the MFMA layout, the scale row of tile row r
    const uint8_t* wrow[RT][2];
    const uint32_t* srow[RT];
    int tile[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        tile[i] = rb * G::TB + wave + 8 * i;
        const RowPtrs lp = resolve_pair<FMT_INT4_FAST, KND>(m.t, min(8 * tile[i] + (lane >> 3), m.t.total_pairs - 1));
        wrow[i][0] = lp.pa + 16 * (lane & 7);
        wrow[i][1] = lp.pb + 16 * (lane & 7);
        const RowPtrs rp = resolve_pair<FMT_INT4_FAST, KND>(m.t, min(8 * tile[i] + (r & 7), m.t.total_pairs - 1));
        srow[i] = (const uint32_t*)(r < 8 ? rp.sa : rp.sb);     // 4-byte aligned rows (even group count)
    }

    // step pair dp of the K block (clamped into it: a pair past the end
    // reloads the last one, whose values are never used)
    const int npairs = nst >> 1;                                  // K blocks hold an even number of steps
    auto load_pair = [&](MfmaRing<NB, PREC>& R, int slot, int dp) {
        const size_t off = (size_t)s0 * 64 + (size_t)min(dp, npairs - 1) * 128;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            R.w[slot][i][0] = ld_g_nt((const u32x4*)(wrow[i][0] + off));
            R.w[slot][i][1] = ld_g_nt((const u32x4*)(wrow[i][1] + off));
        }
    };
    // scales of chunk c: lane (r, q) holds dword q of the chunk's groups of
    // row r (chunks start on an even group)
    const int ngd = m.nsteps >> (m.gshift + 1);                  // scale dwords per row
    auto load_scales = [&](u32 (&sv)[RT], int c) {
        const int d0 = ((s0 + c * SC) >> m.gshift) >> 1;
#pragma unroll
        for (int i = 0; i < RT; ++i) sv[i] = ld_g(srow[i] + min(d0 + q, ngd - 1));
    };

    // staged-activation chunk c of this K block: pieces into registers, then to LDS
    u32x4 pre[G::LPT];
    u32 scn[RT], scc[RT];
    auto chunk_issue = [&](int c) {
#pragma unroll
        for (int i = 0; i < G::LPT; ++i) {
            const int idx = min(tid + i * G::NT, G::CHUNK_LOADS - 1);
            const int row = idx / (SC * 16), piece = idx - row * (SC * 16);     // row = plane * NB + seq
            const int st = min(s0 + c * SC + (piece >> 4), m.nsteps - 1);
            pre[i] = ld_g((const u32x4*)(m.xs + (size_t)row * (K >> 1) + (size_t)st * 64) + (piece & 15));
        }
        load_scales(scn, c);
    };
    auto chunk_write = [&](int buf) {
#pragma unroll
        for (int i = 0; i < G::LPT; ++i) {
            const int idx = tid + i * G::NT;
            if (idx < G::CHUNK_LOADS) {
                const int row = idx / (SC * 16), piece = idx - row * (SC * 16);
                *(u32x4*)(act_buf + buf * G::ACT_B + row * G::ROW_B + piece * 16) = pre[i];
            }
        }
#pragma unroll
        for (int i = 0; i < RT; ++i) scc[i] = scn[i];
    };

    f4 acc[RT][NTL];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int n = 0; n < NTL; ++n) acc[i][n] = f4{0.f, 0.f, 0.f, 0.f};

    MfmaRing<NB, PREC> R;
    chunk_issue(0);
#pragma unroll
    for (int d = 0; d < D; ++d) load_pair(R, d, d);
    chunk_write(0);
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        if (c + 1 < nch) chunk_issue(c + 1);
        const char* ab = act_buf + buf * G::ACT_B;
#pragma unroll
        for (int k = 0; k < SC / 2; ++k) {
            const int dp = c * (SC / 2) + k;
            const int slot = k % D;
            // the step pair's bytes into the MFMA layout
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    *(u32x4*)(wlds + t * G::WT_B + (8 * h + (lane >> 3)) * G::WROW_B + (lane & 7) * 16) = R.w[slot][t][h];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int i = 2 * k + s;                      // step within the chunk
                if (c * SC + i < nst) {
                    const int rel = i >> m.gshift;            // group within the chunk
                    const int src = r + 16 * (rel >> 1);
                    float sc[RT];
                    h8 bw[RT][4];
#pragma unroll
                    for (int t = 0; t < RT; ++t) {
                        const u32 sw = (u32)__shfl((int)scc[t], src, 64);
                        sc[t] = __uint_as_float((rel & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
                        const u32x4 wv = *(const u32x4*)(wlds + t * G::WT_B + r * G::WROW_B + (4 * s + q) * 16);
                        bw[t][0] = unpack_b(wv.x);
                        bw[t][1] = unpack_b(wv.y);
                        bw[t][2] = unpack_b(wv.z);
                        bw[t][3] = unpack_b(wv.w);
                    }
#pragma unroll
                    for (int n = 0; n < NTL; ++n) {
                        f4 cg[RT];
#pragma unroll
                        for (int t = 0; t < RT; ++t) cg[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
#pragma unroll
                            for (int p = 0; p < PREC; ++p) {
                                const h8 a = *(const h8*)(ab + (p * NB + n * 16 + r) * G::ROW_B + (i * 128 + 32 * q + 8 * j) * 2);
#pragma unroll
                                for (int t = 0; t < RT; ++t) cg[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bw[t][j], cg[t], 0, 0, 0);
                            }
                        }
#pragma unroll
                        for (int t = 0; t < RT; ++t) {
                            acc[t][n].x = fmaf(sc[t], cg[t].x, acc[t][n].x);
                            acc[t][n].y = fmaf(sc[t], cg[t].y, acc[t][n].y);
                            acc[t][n].z = fmaf(sc[t], cg[t].z, acc[t][n].z);
                            acc[t][n].w = fmaf(sc[t], cg[t].w, acc[t][n].w);
                        }
                    }
                }
            }
            load_pair(R, slot, dp + D);
        }
        if (c + 1 < nch) chunk_write(buf ^ 1);
        __syncthreads();
    }

    if constexpr (EK == MEPI_ARGMAX) {
        // K is never split on this path: per lane keys of its 4*NTL sequences
        u64 best[NTL][4];
#pragma unroll
        for (int n = 0; n < NTL; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) best[n][e] = 0ull;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int pair = 8 * tile[t] + (r & 7);
            const int row = 2 * pair + (r >> 3);          // adjacent-row pairs (LM head)
            const bool ok = pair < m.t.total_pairs && row < m.t.a.n;
#pragma unroll
            for (int n = 0; n < NTL; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int seq = n * 16 + 4 * q + e;      // padded sequences (seq >= nb) keep key 0
                    const u64 k = (ok && seq < m.nb)
                                      ? argmax_key(epi.score(acc[t][n][e] * ld_g(m.xscale + seq), seq, (u32)row), (u32)row)
                                      : 0ull;
                    best[n][e] = k > best[n][e] ? k : best[n][e];
                }
        }
        // max over the 16 rows of the lane group, then over waves
#pragma unroll
        for (int n = 0; n < NTL; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u64 k = best[n][e];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    const u32 lo = __shfl_xor((u32)k, o, 64), hi = __shfl_xor((u32)(k >> 32), o, 64);
                    const u64 k2 = ((u64)hi << 32) | lo;
                    k = k2 > k ? k2 : k;
                }
                if (r == 0) key_lds[wave * NB + n * 16 + 4 * q + e] = k;
            }
        __syncthreads();
        if (tid < NB) {
            u64 b = 0;
            for (int w = 0; w < G::NT / 64; ++w) b = key_lds[w * NB + tid] > b ? key_lds[w * NB + tid] : b;
            wg_keys[(size_t)blockIdx.x * NB + tid] = b;
        }
    } else if (m.kb == 1) {
        // the two rows of a pair are in lanes r and r ^ 8
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int n = 0; n < NTL; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = acc[t][n][e];
                    const float o = shfl_xor_f(v, 8);
                    const int pair = 8 * tile[t] + r;
                    const int b = n * 16 + 4 * q + e;
                    if (r < 8 && pair < m.t.total_pairs && b < m.nb) {
                        const float xsc = ld_g(m.xscale + b);
                        epi(0, pair, b, v * xsc, o * xsc);
                    }
                }
    } else {
        // K split: partials through to memory, the last workgroup of the row
        // block to arrive adds them in K-block order
#pragma unroll
        for (int t = 0; t < RT; ++t)
            if (tile[t] < m.tiles) {
                float* pp = m.part + ((size_t)tile[t] * m.kb + kbi) * NB * 16;
#pragma unroll
                for (int n = 0; n < NTL; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) st_dev(pp + (n * 16 + 4 * q + e) * 16 + r, acc[t][n][e]);
            }
        wait_stores();
        __syncthreads();
        if (tid == 0) {
            int* c = m.cnt + rb;
            const int old = __hip_atomic_fetch_add((I4D_GLOBAL int*)c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int is_last = (old == m.kb - 1);
            if (is_last) st_dev(c, 0);                  // ready for the next call
            flag[0] = is_last;
        }
        __syncthreads();
        if (flag[0]) {
            const int t0 = rb * G::TB;
            const int ntl = min(G::TB, m.tiles - t0);
            for (int idx = tid; idx < ntl * m.nb * 8; idx += G::NT) {
                const int tl = idx / (m.nb * 8), rem = idx - tl * (m.nb * 8);
                const int b = rem >> 3, mm = rem & 7;
                const int pair = 8 * (t0 + tl) + mm;
                const float* pp = m.part + (size_t)(t0 + tl) * m.kb * NB * 16 + b * 16 + mm;
                float va = 0.f, vb = 0.f;
                for (int k = 0; k < m.kb; ++k) {
                    va += ld_g(pp + (size_t)k * NB * 16);
                    vb += ld_g(pp + (size_t)k * NB * 16 + 8);
                }
                const float xsc = ld_g(m.xscale + b);
                if (pair < m.t.total_pairs) epi(0, pair, b, va * xsc, vb * xsc);
            }
        }
    }
}
