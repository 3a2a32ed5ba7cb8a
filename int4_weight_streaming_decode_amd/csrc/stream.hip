// Streaming decode kernel: one persistent launch runs every layer of a
// batch-1 decode step (gfx950, wave64).
//
// Why one launch.  At batch 1 every weight byte is read once per token and the
// step is bound by HBM (Primer 1.2; Roofline reply 一/二).  Issued as one kernel
// per phase, each of the five phases of a layer pays its own start-up (the
// first weight bytes arrive only after the activations are staged) and its own
// drain; the pages' cure is fusion so that nothing stops the weight stream
// (Unsloth article 二.1, Roofline reply 三).  Here one workgroup per compute
// unit walks all phases of all layers, and its weight stream never stops at a
// phase boundary (weights do not depend on activations).
//
// Two roles per workgroup.  Two of its ten waves only move weights: they
// walk the units of every phase of every layer in order and copy them into a
// ring in LDS, as far ahead as the ring allows.  The other eight waves stage
// the activations, take the exchange waits, form the dot products from the
// ring and run attention and the epilogues.  A wave's vector-memory loads
// complete in issue order, so a wave that both prefetched weights and waited
// for an exchange value would wait for its prefetch as well; with the roles
// in different waves, the weight stream runs on through every exchange wait,
// staging and epilogue until the ring is full.
//
// Exchange between workgroups.  Every value one workgroup hands to another
// (q, the new k/v, attention partials, merged heads, residual stream, SwiGLU
// activations) is stored as a 64-bit word: the fp32 value and a 32-bit tag
// that is unique to this launch.  A reader loads the words -- plainly first,
// so the 32 compute units of an XCD share one fetch through their L2 -- and
// reloads any word whose tag is stale with device-scope loads until it is
// current.  There is no grid barrier and no write acknowledgement on the
// critical path: a value is usable as soon as its own word arrives.  Each
// layer has its own exchange region, so a plain load never meets a line that
// was cached earlier in the same launch.
//
// The int4 dot product.  Activations are staged in LDS as integers: each run
// of 32 inputs is scaled by a power of two so that its largest magnitude lies
// in [2^13, 2^14), rounded to an integer a, and a is written as four balanced
// base-16 digits d_p in [-8, 7] (a = sum_p d_p 16^p; the nibbles of
// (a + 0x8888) ^ 0x8888).  Plane p holds digit p of every input, eight inputs
// per dword in the weight codes' nibble order.  A code dword XOR 0x88888888
// is the eight signed int4 values c - 8, so v_dot8_i32_i4 against plane p
// gives sum (c - 8) d_p exactly; the four plane sums are combined by shifts
// into sum (c - 8) a (exact in int32), converted once, and scaled by the
// group scale times the run's power of two.  The only rounding is that of the
// activations to 15 significant bits relative to their run's maximum (23 bits
// and six digit planes for the k and v rows, which are rounded to bf16 into
// the cache), and no activation can overflow (the power of two adapts to any
// finite value).
// About 0.85 VALU operations per weight.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>

#include "stream.h"
#include "attention.h"
#include "common.h"

namespace i4d_stream {
namespace {

constexpr int NT = 640;            // threads per workgroup: 10 waves, eight consumers (two per SIMD) and two loaders
constexpr int NWAVE = NT / 64;
constexpr int NLW = 2;             // loader waves: they only copy weights from HBM into the LDS ring
constexpr int NCW = NWAVE - NLW;   // consumer waves: staging, exchange, dot products, attention, epilogues
constexpr int NCT = NCW * 64;      // consumer threads (thread ids 0 .. NCT - 1)
constexpr int CPL = NCW / NLW;     // consumer waves fed by one loader wave
constexpr int NSLOT = NCT / 16;    // 16-lane slots of the consumers
constexpr int SPL = NSLOT / NLW;   // slots fed by one loader wave
static_assert(SPL == 4 * CPL && NLW * CPL == NCW, "a loader wave feeds whole consumer waves");
// One step of one loader's half of the ring: for each of its consumer waves,
// 1 KB of row-a codes and 1 KB of row-b codes (16 bytes per consumer lane),
// then the two scale words of each row of each of its slots.
constexpr int HSTEP = CPL * 2 * 1024 + SPL * 16;
constexpr int LDEPTH = 3;          // steps a loader wave keeps in flight (registers)
constexpr int NBMAX = 16;          // ring steps at most
constexpr int HD = 128;
constexpr int ANSW = 2;            // attention subtiles per wave per load round
constexpr int MAXRUN = 8;          // pair runs per slot per phase
constexpr int MAX_LAYERS = 128;    // layer table kept in LDS
constexpr int MAX_RES = 64;        // residual rows per compute unit: pairs of Wo / W_down
constexpr int KMAX = 32768;        // largest K
constexpr int RMN = 2;             // staging rounds of NCT groups of 8 for K <= 8192 (d_model, q width)
constexpr int RMD = 5;             // staging rounds per pass for W_down's input (d_ff <= 20480: one pass)
constexpr int SPIN_LIMIT = 1 << 17;   // polls of an exchange word
constexpr int WAIT_LIMIT = 1 << 23;   // polls of a wait between the waves of one workgroup

enum { K_QKV = 0, K_WO = 1, K_GU = 2, K_DN = 3 };

// ------------------------------------------------------------------ layer table
struct LPtr {
    const uint8_t* c[7];          // codes of wq wk wv wo wg wu wd
    const uint8_t* s[7];          // their bf16 scales (byte pointers)
    const uint16_t* g1;           // attention norm gain
    const uint16_t* g2;           // FFN norm gain
    uint16_t* kc;
    uint16_t* vc;
};
constexpr int LPTR_WORDS = (int)(sizeof(LPtr) / 8);

// ------------------------------------------------------------------ per-kind geometry (same for every layer)
// A phase streams pairs of rows: q/k/v (i, i + hd/2) of one head of ONE of
// the three matrices (compute units are split between q, k and v in
// proportion to their rows); Wo and W_down rows (p, p + D/2); gate row p with
// up row p.  The pairs of a compute unit are cut into units of 16 lanes x 16
// bytes per row (512 inputs) and the units into one contiguous range per
// 16-lane slot; every slot runs n steps (a short range skips its last ones).
struct KGeo {
    int S;                        // units per row (K / 512)
    int K;
    int p0, np;                   // this unit's first pair and pair count (within its matrix)
    int U, n;                     // units, steps per slot
    int mia, mib;                 // table index of the matrix of row a, row b
    int mat;                      // q/k/v: 0, 1, 2
    unsigned ca_off, cb_off;      // code byte offsets of pair p0's rows a and b
    unsigned sa_off, sb_off;      // scale byte offsets
    unsigned jump;                // q/k/v: extra code advance at a head boundary
    int jper;                     // units between head boundaries (0: none)
};
// The scale byte offset of a unit is its code byte offset / 32 (two bytes of
// scale per 64 bytes of codes), so the loader only tracks the latter.
struct SGeo {                     // per (kind, slot)
    int len, seg0, cnt0, u0, pair0;   // pair0: local index of the slot's first pair
    unsigned off0;                // byte offset of the slot's first unit in its code stream (lane 0)
};

struct Args {
    const LPtr* table;
    int L;
    const float* x_in;
    float* x_out;
    const int* pos;
    int max_pos, cap;
    int D, F, Hq, Hkv;
    float eps, qscale;
    double base;
    int nsplit;                    // attention: splits per KV head
    int cq, ck;                    // compute units [0, cq): q rows, [cq, ck): k rows, [ck, nwg): v rows
    int ps, nb;                    // LDS bytes per digit plane; ring steps
    unsigned off_act, off_ring;    // LDS offsets of the staging / attention area and of the ring
    char* lbase;                   // exchange regions: lbase + l * lstride
    size_t lstride;
    unsigned ox, oq, okv, opart, oo, oy, oact;   // byte offsets in a region
    const uint8_t* zero;           // 1 KB of zeros (loads past the last phase)
    int* status;
    unsigned* epoch;
};

// ------------------------------------------------------------------ LDS layout
// Fixed part first; then the layer table; then (offsets per launch, from the
// shapes) the staging area -- digit planes and run scales, or attention's and
// the merge's working set -- and the weight ring, NLW halves of nb steps.
constexpr int ATT_LDS = NCW * (16 * HD + 32) * 4 + (HD / 16) * 2 * 64 * 8;   // attn_lds_bytes<HD, NCT>
constexpr int MERGE_LDS = (64 + 64 + 64 * 32) * 4;
constexpr int OFF_PART = 0;                                        // float2 [NSLOT][MAXRUN]
constexpr int OFF_RES = OFF_PART + NSLOT * MAXRUN * 8;             // float [4][MAX_RES]: x rows a, b; y rows a, b
constexpr int OFF_ROPE = OFF_RES + 4 * MAX_RES * 4;                // float2 [HD / 2]
constexpr int OFF_KG = OFF_ROPE + (HD / 2) * 8;                    // KGeo [4]
constexpr int OFF_SG = OFF_KG + 4 * (int)sizeof(KGeo);             // SGeo [4][NSLOT]
constexpr int OFF_RED = OFF_SG + 4 * NSLOT * (int)sizeof(SGeo);    // float [NCW] (+ NCW unused)
constexpr int MAXNP = (MAXRUN - 1) * NSLOT;                        // pairs per unit and phase (runs_of() <= MAXRUN)
constexpr int OFF_PINFO = OFF_RED + 2 * NCW * 4;                   // u32 [4][MAXNP]: first entry << 8 | count
constexpr int OFF_PLIST = OFF_PINFO + 4 * MAXNP * 4;               // u8 [4][NSLOT * MAXRUN]: part indices, pair-major
constexpr int OFF_SYNC = ((OFF_PLIST + 4 * NSLOT * MAXRUN + 15) / 16) * 16;   // u32 [16], see below
constexpr int OFF_TAB = ((OFF_SYNC + 64 + 255) / 256) * 256;       // LPtr [L]
// words of the sync block
constexpr int SY_READY = 0;        // [NLW]: steps the loader wave has written into its half
constexpr int SY_CONS = 4;         // [NCW]: steps the consumer wave has read
constexpr int SY_BAR = 12;         // arrivals at the consumers' barriers
constexpr int SY_ABORT = 13;       // set by a wave that gave up an intra-workgroup wait

// ------------------------------------------------------------------ helpers
typedef u64 u64x2 __attribute__((ext_vector_type(2)));

template <class T> I4D_DEVINL T* uni(T* p) {        // a pointer every lane holds equally, in scalar registers
    const u64 v = (u64)p;
    const u32 lo = __builtin_amdgcn_readfirstlane((u32)v), hi = __builtin_amdgcn_readfirstlane((u32)(v >> 32));
    return (T*)(((u64)hi << 32) | lo);
}
I4D_DEVINL int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
I4D_DEVINL unsigned uniu(unsigned v) { return (unsigned)__builtin_amdgcn_readfirstlane((int)v); }

// An opaque copy of the pointer to the launch arguments, in the constant
// address space: fields read through it are re-read (scalar loads) where
// they are used instead of being hoisted out of the layer loop into registers
// that would stay live across every phase.
template <class T> I4D_DEVINL const I4D_CONST T* opaque_ptr(const T* p) {
    const I4D_CONST T* c = (const I4D_CONST T*)p;
    asm volatile("" : "+s"(c));
    return c;
}

// Base of layer l's exchange region, from an opaque read of the arguments.
I4D_DEVINL char* layer_region(const struct Args* Ap, int l) {
    const I4D_CONST Args& a = *opaque_ptr(Ap);
    return a.lbase + (size_t)l * a.lstride;
}

I4D_DEVINL void ll_put(u64* p, float v, u32 tag) { st_dev_t(p, ((u64)tag << 32) | (u64)__float_as_uint(v)); }

struct Spin {
    int* status;
    bool dead;                   // this thread gave up waiting once: it no longer waits
};

// N consecutive exchange words from p (16-byte aligned, N even): plain loads,
// then device-scope reloads of every word whose tag is not `tag` (bounded).
template <int N>
I4D_DEVINL void ll_get(const u64* p, u32 tag, float (&v)[N], Spin& sp) {
    u64 w[N];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const u64x2 t = ld_g((const u64x2*)p + i);
        w[2 * i] = t.x;
        w[2 * i + 1] = t.y;
    }
    int polls = 0;
    for (;;) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < N; ++i) ok = ok && (u32)(w[i] >> 32) == tag;
        if (ok || sp.dead) break;
        if (++polls > SPIN_LIMIT) {
            sp.dead = true;
            raise_status(sp.status, I4D_DEV_BARRIER_TIMEOUT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int i = 0; i < N; ++i)
            if ((u32)(w[i] >> 32) != tag) w[i] = ld_dev_t(p + i);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __uint_as_float((u32)w[i]);
}

// The wide activations (o, y, act) travel as packed 32-bit words: the fp32
// value rounded to 15 mantissa bits (round to nearest even; the staging keeps
// 15 bits relative to each 32-input run's largest value anyway) in the upper
// 24 bits, the low 8 bits of the launch tag below (a word left by an earlier
// launch carries another tag byte).
I4D_DEVINL u32 pk_word(float v, u32 tag) {
    u32 u = __float_as_uint(v);
    u += 0x7Fu + ((u >> 8) & 1u);
    return (u & 0xFFFFFF00u) | (tag & 0xFFu);
}
I4D_DEVINL void pk_put(u32* p, float v, u32 tag) { st_dev_t(p, pk_word(v, tag)); }
I4D_DEVINL float pk_val(u32 w) { return __uint_as_float(w & 0xFFFFFF00u); }

// This consumer thread's input groups g = g0 + tid + r * NCT (r < RM; groups
// past ngr read the last group again) from an exchange vector: first a
// device-scope wait for the last word of the thread's last group, then plain
// loads of all its groups (one memory round trip for the lot), then
// device-scope reloads of the words whose tag is not yet current, until every
// tag is (bounded).  The first wait keeps the plain loads from running ahead
// of most producers: a plain load of a line not yet written leaves that stale
// line in the L2, where the other compute units of the XCD then find it and
// must reload.
// WIDE: 64-bit words (value, 32-bit tag); otherwise packed 32-bit words.
template <int RM, bool WIDE>
I4D_DEVINL void fetch_groups(const void* src, int g0, int ngr, u32 tag, float (&v)[RM][8], Spin& sp) {
    const int tid = i4d_tid();
    {
        // two polls in flight, half a round trip apart: the word is seen about a
        // quarter of a round trip sooner than with one poll at a time
        const int gl = min(g0 + tid + (RM - 1) * NCT, ngr - 1);
        auto poll = [&]() -> u32 {
            if constexpr (WIDE) return (u32)(ld_dev_t((const u64*)src + 8 * (size_t)gl + 7) >> 32);
            else return ld_dev_t((const u32*)src + 8 * (size_t)gl + 7);
        };
        auto ok = [&](u32 w) { return WIDE ? w == tag : (w & 0xFFu) == (tag & 0xFFu); };
        if (!sp.dead) {
            u32 w0 = poll();
            __builtin_amdgcn_s_sleep(8);
            u32 w1 = poll();
            for (int polls = 0;; polls += 2) {
                if (ok(w0)) break;
                w0 = poll();
                if (ok(w1)) break;
                w1 = poll();
                if (polls > SPIN_LIMIT) {
                    sp.dead = true;
                    raise_status(sp.status, I4D_DEV_BARRIER_TIMEOUT);
                    break;
                }
            }
        }
    }
    if constexpr (WIDE) {
        const u64* p = (const u64*)src;
        u64 w[RM][8];
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const int g = min(g0 + tid + r * NCT, ngr - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u64x2 t = ld_g((const u64x2*)(p + 8 * (size_t)g) + i);
                w[r][2 * i] = t.x; w[r][2 * i + 1] = t.y;
            }
        }
        for (int polls = 0;;) {
            bool ok = true;
#pragma unroll
            for (int r = 0; r < RM; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) ok = ok && (u32)(w[r][e] >> 32) == tag;
            if (ok || sp.dead) break;
            if (++polls > SPIN_LIMIT) { sp.dead = true; raise_status(sp.status, I4D_DEV_BARRIER_TIMEOUT); break; }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const int g = min(g0 + tid + r * NCT, ngr - 1);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((u32)(w[r][e] >> 32) != tag) w[r][e] = ld_dev_t(p + 8 * (size_t)g + e);
            }
        }
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[r][e] = __uint_as_float((u32)w[r][e]);
    } else {
        const u32* p = (const u32*)src;
        const u32 t8 = tag & 0xFFu;
        u32 w[RM][8];
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const int g = min(g0 + tid + r * NCT, ngr - 1);
            const u32x4 a = ld_g((const u32x4*)(p + 8 * (size_t)g)), b = ld_g((const u32x4*)(p + 8 * (size_t)g) + 1);
            w[r][0] = a.x; w[r][1] = a.y; w[r][2] = a.z; w[r][3] = a.w;
            w[r][4] = b.x; w[r][5] = b.y; w[r][6] = b.z; w[r][7] = b.w;
        }
        for (int polls = 0;;) {
            bool ok = true;
#pragma unroll
            for (int r = 0; r < RM; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) ok = ok && (w[r][e] & 0xFFu) == t8;
            if (ok || sp.dead) break;
            if (++polls > SPIN_LIMIT) { sp.dead = true; raise_status(sp.status, I4D_DEV_BARRIER_TIMEOUT); break; }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const int g = min(g0 + tid + r * NCT, ngr - 1);
#pragma unroll
                for (int e = 0; e < 8; e += 2)
                    if ((w[r][e] & 0xFFu) != t8 || (w[r][e + 1] & 0xFFu) != t8) {
                        const u64 t = ld_dev_t((const u64*)(p + 8 * (size_t)g + e));
                        w[r][e] = (u32)t; w[r][e + 1] = (u32)(t >> 32);
                    }
            }
        }
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[r][e] = pk_val(w[r][e]);
    }
}

// ------------------------------------------------------------------ waits between the waves of one workgroup
// LDS words written by one wave and polled by another.  LDS executes the
// operations of one wave in issue order, so a word written after some data is
// seen only after that data; the signal fences keep the compiler from moving
// memory operations across the hand-off.  Every wait is bounded: a wave that
// gives up raises I4D_DEV_BARRIER_TIMEOUT and sets the abort word, after
// which no wave of the workgroup waits any more (results are then wrong, but
// the launch ends).
#define I4D_LDS __attribute__((address_space(3)))
I4D_DEVINL u32 lds_get(const u32* p) { return uniu(*(const volatile I4D_LDS u32*)p); }
I4D_DEVINL void lds_put(u32* p, u32 v) { *(volatile I4D_LDS u32*)p = v; }

// Wait until f() (a re-read of some LDS words) reaches `need`; returns the last value read.
template <class F>
I4D_DEVINL u32 lds_wait(F f, u32 need, u32* sync, int* status) {
    u32 v = f();
    for (int polls = 0; (int)(v - need) < 0; ) {
        if (lds_get(sync + SY_ABORT)) break;
        if (++polls > WAIT_LIMIT) {
            lds_put(sync + SY_ABORT, 1u);
            if ((i4d_tid() & 63) == 0) raise_status(status, I4D_DEV_BARRIER_TIMEOUT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = f();
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return v;
}

// A barrier of the NCW consumer waves only (the loader waves never stop for
// one): each wave adds one arrival and waits for all arrivals of this barrier.
struct CBar {
    u32* sync;
    int* status;
    u32 target;                  // arrivals that complete this wave's next barrier
};
I4D_DEVINL void cbar(CBar& b) {
    __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0): this wave's LDS writes have landed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if ((i4d_tid() & 63) == 0)
        __hip_atomic_fetch_add((I4D_LDS u32*)(b.sync + SY_BAR), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    b.target += NCW;
    u32* s = b.sync;
    (void)lds_wait([&] { return lds_get(s + SY_BAR); }, b.target, s, b.status);
}

// ------------------------------------------------------------------ the loader waves
// One loader lane copies, per step, the 16 bytes of row a and of row b that
// consumer lane `lane` of each of its CPL consumer waves will use, and one
// scale word (lanes < 4 * SPL).  Loads go through buffer descriptors built
// once per phase (scalar base, 32-bit lane offset), and a slot's offset at
// step j is computed from j alone: its first unit's offset, 256 bytes per
// unit, and the q/k/v head jump once j reaches the slot's head boundary (a
// slot holds at most MAXRUN * S units, fewer than a head's 64 * S, so it
// crosses at most one).  A step past the slot's range reads the phase's first
// bytes again.
struct LSlot { unsigned off0; int len, jat; };     // jat: first step past the head boundary
struct Loader {
    __amdgpu_buffer_rsrc_t ca, cb;
    const uint8_t* sa; const uint8_t* sb;      // scale rows (a lane picks one: a plain global load)
    unsigned jump;
    int j, n, ph, nph;
    LSlot cs[CPL], ss;
};
struct Stage { u32x4 a[CPL], b[CPL]; u32 s; };

I4D_DEVINL __amdgpu_buffer_rsrc_t rsrc_of(const uint8_t* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)uni(p), (short)0, -1, 0x00020000);
}

I4D_DEVINL void loader_next(Loader& Ld, const KGeo* kg, const SGeo* sg, const LPtr* tab, const uint8_t* zero, int lw) {
    do { ++Ld.ph; } while (Ld.ph < Ld.nph && kg[Ld.ph & 3].n == 0);
    if (Ld.ph >= Ld.nph) {       // past the last phase: reads of a zero block, never consumed
        Ld.ca = Ld.cb = rsrc_of(zero);
        Ld.sa = Ld.sb = uni(zero);
        Ld.n = 0x7FFFFFFF; Ld.j = 0; Ld.jump = 0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) Ld.cs[i] = LSlot{0u, 0, 1 << 30};
        Ld.ss = LSlot{0u, 0, 1 << 30};
        return;
    }
    const int kind = Ld.ph & 3, l = Ld.ph >> 2;
    const KGeo& k = kg[kind];
    const LPtr& t = tab[l];
    Ld.ca = rsrc_of(t.c[k.mia] + k.ca_off);
    Ld.cb = rsrc_of(t.c[k.mib] + k.cb_off);
    Ld.sa = uni(t.s[k.mia] + k.sa_off);
    Ld.sb = uni(t.s[k.mib] + k.sb_off);
    Ld.n = uni(k.n); Ld.j = 0;
    Ld.jump = uniu(k.jump);
    const int lane = i4d_tid() & 63;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const SGeo& s = sg[kind * NSLOT + SPL * lw + 4 * i + (lane >> 4)];
        Ld.cs[i] = LSlot{s.off0 + (unsigned)(lane & 15) * 16u, s.len, s.cnt0};
    }
    const SGeo& s = sg[kind * NSLOT + SPL * lw + min(lane >> 2, SPL - 1)];
    Ld.ss = LSlot{s.off0, s.len, s.cnt0};
}

// Issue the loads of the next step into st (always the same 2 CPL + 1 loads,
// so that the compiler's wait counts stay exact) and advance.
I4D_DEVINL void loader_issue(Loader& Ld, Stage& st, const KGeo* kg, const SGeo* sg, const LPtr* tab, const uint8_t* zero,
                             int lw) {
    if (Ld.j == Ld.n) loader_next(Ld, kg, sg, tab, zero, lw);
    const int lane = i4d_tid() & 63, j = Ld.j;
    const unsigned jo = (unsigned)j << 8;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const LSlot& q = Ld.cs[i];
        const unsigned o = j < q.len ? q.off0 + jo + (j >= q.jat ? Ld.jump : 0u) : (unsigned)(lane & 15) * 16u;
        st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(Ld.ca, (int)o, 0, 2);     // nontemporal
        st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(Ld.cb, (int)o, 0, 2);
    }
    {
        const LSlot& q = Ld.ss;
        const unsigned so = (j < q.len ? (q.off0 + jo + (j >= q.jat ? Ld.jump : 0u)) >> 5 : 0u) + 4u * (unsigned)(lane & 1);
        const size_t ds = ((lane >> 1) & 1) ? (size_t)((uintptr_t)Ld.sb - (uintptr_t)Ld.sa) : 0u;
        st.s = ld_g((const u32*)(Ld.sa + ds + so));
    }
    ++Ld.j;
}

// Loader wave lw: every step of every phase of every layer, LDEPTH steps in
// flight in registers; step t goes into ring entry t mod nb of its half once
// every consumer wave of the half has read the step that entry held.
I4D_DEVINL void loader_main(const I4D_CONST Args& A, const KGeo* kg, const SGeo* sg, const LPtr* tab, char* ring,
                            u32* sync, int lw) {
    const int lane = i4d_tid() & 63;
    const int nb = uni(A.nb);
    char* half = ring + (size_t)lw * nb * HSTEP;
    u32* ready = sync + SY_READY + lw;
    const u32* cons = sync + SY_CONS + CPL * lw;
    const int T = uni(A.L * (kg[0].n + kg[1].n + kg[2].n + kg[3].n));
    Loader Ld;
    Ld.ph = -1; Ld.nph = 4 * A.L; Ld.j = 0; Ld.n = 0;
    Stage st[LDEPTH];
#pragma unroll
    for (int i = 0; i < LDEPTH; ++i) loader_issue(Ld, st[i], kg, sg, tab, A.zero, lw);
    auto cmin = [&] {
        u32 m = lds_get(cons);
#pragma unroll
        for (int i = 1; i < CPL; ++i) m = min(m, lds_get(cons + i));
        return m;
    };
    u32 freed = 0;                  // steps every consumer wave of the half has read (last seen)
    int slot = 0;
    for (int t0 = 0; t0 < T; t0 += LDEPTH) {
#pragma unroll
        for (int i = 0; i < LDEPTH; ++i) {
            const int t = t0 + i;
            if (t < T) {
                if ((int)freed < t - nb + 1) freed = lds_wait(cmin, (u32)(t - nb + 1), sync, A.status);
                char* dst = half + slot * HSTEP;
#pragma unroll
                for (int q = 0; q < CPL; ++q) {
                    *(u32x4*)(dst + (2 * q) * 1024 + lane * 16) = st[i].a[q];
                    *(u32x4*)(dst + (2 * q + 1) * 1024 + lane * 16) = st[i].b[q];
                }
                if (lane < 4 * SPL) *(u32*)(dst + CPL * 2048 + lane * 4) = st[i].s;
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                if (lane == 0) lds_put(ready, (u32)(t + 1));
                slot = slot + 1 == nb ? 0 : slot + 1;
            }
            loader_issue(Ld, st[i], kg, sg, tab, A.zero, lw);
        }
    }
}

// ------------------------------------------------------------------ the dot product of one unit
// sum of the eight signed 4-bit products of w and d, starting from zero: the
// three-operand form takes the zero as an inline constant (the compiler would
// otherwise zero a register for the two-operand form that accumulates in place)
I4D_DEVINL int dot8_first(int w, int d) {
    int r;
    asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(w), "v"(d));
    return r;
}

// Digit planes 0..3 at act + p * ps; for the q/k/v projection (six planes,
// K = d_model <= ps, so each plane fills at most half of its slot) planes 4
// and 5 sit in the upper halves of slots 0 and 1.
struct Unit { u32x4 a, b; u32 sa, sb; };

I4D_DEVINL void dot_unit(const Unit& u, const char* act, int ps, unsigned aoff, float cs, int hs, bool six, float& ra,
                         float& rb) {
    const char* ap = act + aoff;
    const u32x4 d0 = *(const u32x4*)(ap);
    const u32x4 d1 = *(const u32x4*)(ap + ps);
    const u32x4 d2 = *(const u32x4*)(ap + 2 * ps);
    const u32x4 d3 = *(const u32x4*)(ap + 3 * ps);
    int a0, a1, a2, a3, b0, b1, b2, b3;
    {
        const int wa = (int)(u.a[0] ^ 0x88888888u), wb = (int)(u.b[0] ^ 0x88888888u);
        a0 = dot8_first(wa, (int)d0[0]); a1 = dot8_first(wa, (int)d1[0]);
        a2 = dot8_first(wa, (int)d2[0]); a3 = dot8_first(wa, (int)d3[0]);
        b0 = dot8_first(wb, (int)d0[0]); b1 = dot8_first(wb, (int)d1[0]);
        b2 = dot8_first(wb, (int)d2[0]); b3 = dot8_first(wb, (int)d3[0]);
    }
#pragma unroll
    for (int q = 1; q < 4; ++q) {
        const int wa = (int)(u.a[q] ^ 0x88888888u), wb = (int)(u.b[q] ^ 0x88888888u);
        a0 = __builtin_amdgcn_sdot8(wa, (int)d0[q], a0, false);
        a1 = __builtin_amdgcn_sdot8(wa, (int)d1[q], a1, false);
        a2 = __builtin_amdgcn_sdot8(wa, (int)d2[q], a2, false);
        a3 = __builtin_amdgcn_sdot8(wa, (int)d3[q], a3, false);
        b0 = __builtin_amdgcn_sdot8(wb, (int)d0[q], b0, false);
        b1 = __builtin_amdgcn_sdot8(wb, (int)d1[q], b1, false);
        b2 = __builtin_amdgcn_sdot8(wb, (int)d2[q], b2, false);
        b3 = __builtin_amdgcn_sdot8(wb, (int)d3[q], b3, false);
    }
    int ia = ((a3 * 16 + a2) * 16 + a1) * 16 + a0;
    int ib = ((b3 * 16 + b2) * 16 + b1) * 16 + b0;
    if (six) {
        const u32x4 d4 = *(const u32x4*)(ap + ps / 2);
        const u32x4 d5 = *(const u32x4*)(ap + ps + ps / 2);
        int a4, a5, b4, b5;
        {
            const int wa = (int)(u.a[0] ^ 0x88888888u), wb = (int)(u.b[0] ^ 0x88888888u);
            a4 = dot8_first(wa, (int)d4[0]); a5 = dot8_first(wa, (int)d5[0]);
            b4 = dot8_first(wb, (int)d4[0]); b5 = dot8_first(wb, (int)d5[0]);
        }
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            const int wa = (int)(u.a[q] ^ 0x88888888u), wb = (int)(u.b[q] ^ 0x88888888u);
            a4 = __builtin_amdgcn_sdot8(wa, (int)d4[q], a4, false);
            a5 = __builtin_amdgcn_sdot8(wa, (int)d5[q], a5, false);
            b4 = __builtin_amdgcn_sdot8(wb, (int)d4[q], b4, false);
            b5 = __builtin_amdgcn_sdot8(wb, (int)d5[q], b5, false);
        }
        // |sum (c - 8) a| < 32 * 8 * 2^22 = 2^30: exact in int32 (the Horner
        // steps may wrap, the two's-complement result does not)
        ia = (int)((u32)(a5 * 16 + a4) * 65536u + (u32)ia);
        ib = (int)((u32)(b5 * 16 + b4) * 65536u + (u32)ib);
    }
    const float sa = __uint_as_float((u.sa << hs) & 0xFFFF0000u);
    const float sb = __uint_as_float((u.sb << hs) & 0xFFFF0000u);
    ra = fmaf((float)ia, sa * cs, ra);
    rb = fmaf((float)ib, sb * cs, rb);
}

// ------------------------------------------------------------------ activation staging
// Eight inputs of group g (inputs 8g..8g+7), already normalised: digits into
// the four planes, the power of two of the 32-input run (a quad of lanes) into
// cs.  Non-finite inputs become zeros and raise I4D_DEV_NONFINITE.
I4D_DEVINL void digitize8(char* act, int ps, float* cs, int g, float (&v)[8], bool six, int* status) {
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    m = fmaxf(m, shfl_xor_f(m, 1));
    m = fmaxf(m, shfl_xor_f(m, 2));
    if (!(m <= 3.0e38f)) {           // inf or NaN somewhere in the run
        if ((i4d_tid() & 3) == 0) raise_status(status, I4D_DEV_NONFINITE);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
        m = 0.f;
    }
    int ex;
    (void)frexpf(m, &ex);            // m < 2^ex (m = 0: ex = 0)
    // four planes: |a| <= 2^14, digits of a + 0x8888; six: |a| <= 2^22, of a + 0x888888
    const int sh = (six ? 22 : 14) - ex;
    const u32 bias = six ? 0x888888u : 0x8888u;
    // a = round-to-nearest-even(v 2^sh), |v 2^sh| < 2^22: adding 1.5 * 2^23 leaves
    // a in the low bits of the sum's encoding (at a = +-2^22 the sum is 2^24 or
    // 2^23, whose encodings still differ from that of 1.5 * 2^23 by exactly a)
    u32 dg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const u32 r = __float_as_uint(ldexpf(v[e], sh) + 12582912.0f);
        dg[e] = (r + (bias - 0x4B400000u)) ^ bias;             // (a + bias) ^ bias: digit p in nibble p
    }
    // plane q = nibble q of dg[0..7] in nibbles 0..7: byte b of the even and of
    // the odd inputs gathered into two words (byte permutes); the low nibbles
    // of those bytes are plane 2b, the high nibbles plane 2b + 1, even/odd
    // interleaved.  perm(x, y, s): result byte k = byte s_k of (x:y), 0-3 from y.
    auto gather = [&](u32 d0, u32 d2, u32 d4, u32 d6, u32 (&w)[3]) {
        const u32 lo02 = __builtin_amdgcn_perm(d2, d0, 0x05010400u), lo46 = __builtin_amdgcn_perm(d6, d4, 0x05010400u);
        w[0] = __builtin_amdgcn_perm(lo46, lo02, 0x05040100u);        // byte 0 of d0 d2 d4 d6
        w[1] = __builtin_amdgcn_perm(lo46, lo02, 0x07060302u);        // byte 1
        if (six) {
            const u32 hi02 = __builtin_amdgcn_perm(d2, d0, 0x07030602u), hi46 = __builtin_amdgcn_perm(d6, d4, 0x07030602u);
            w[2] = __builtin_amdgcn_perm(hi46, hi02, 0x05040100u);    // byte 2
        } else {
            w[2] = 0u;
        }
    };
    u32 ev[3], od[3];
    gather(dg[0], dg[2], dg[4], dg[6], ev);
    gather(dg[1], dg[3], dg[5], dg[7], od);
    u32 pl[6];
#pragma unroll
    for (int b = 0; b < 3; ++b) {
        pl[2 * b] = (ev[b] & 0x0F0F0F0Fu) | ((od[b] << 4) & 0xF0F0F0F0u);
        pl[2 * b + 1] = ((ev[b] >> 4) & 0x0F0F0F0Fu) | (od[b] & 0xF0F0F0F0u);
    }
    char* p = act + 4 * g;
    *(u32*)(p) = pl[0];
    *(u32*)(p + ps) = pl[1];
    *(u32*)(p + 2 * ps) = pl[2];
    *(u32*)(p + 3 * ps) = pl[3];
    if (six) {
        *(u32*)(p + ps / 2) = pl[4];
        *(u32*)(p + ps + ps / 2) = pl[5];
    }
    if ((i4d_tid() & 3) == 0) cs[g >> 2] = ldexpf(1.f, -sh);
}

// This consumer wave's sum of v into red[wave]; the reader waits for a
// consumer barrier first.  red[] is written by the two normalised stagings of
// a layer (q/k/v, gate/up) and read by the same phase's epilogue; between a
// phase's epilogue and the next staging that writes red[] lies at least one
// consumer barrier that every wave reaches only after its epilogue.
I4D_DEVINL void wave_share(float v, float* red) {
    for (int o = 32; o >= 1; o >>= 1) v += shfl_xor_f(v, o);
    if ((i4d_tid() & 63) == 0) red[i4d_tid() >> 6] = v;
}

// ------------------------------------------------------------------ attention item of a compute unit
// Item c = (KV head j, split s) of layer l at this launch's position p (-1 if
// invalid).  Splits hold whole 16-key tiles of the cached keys 0 .. p - 1; the
// new key p joins the split that holds it, or the last one when p falls just
// past them (p a multiple of nsplit * 16): its K and V come from the exchange,
// so that extra subtile needs no load.
I4D_DEVINL void attn_setup(const I4D_CONST Args& A, const LPtr* tab, int l, int c, int p, AttnArgs& a, AttnGeo& g) {
    memset(&a, 0, sizeof(a));
    a.kc = tab[l].kc; a.vc = tab[l].vc; a.pos = A.pos;
    a.cap = A.cap; a.hq = A.Hq; a.hkv = A.Hkv; a.batch = 1; a.max_pos = A.max_pos;
    a.kvb = 1; a.nsplit = A.nsplit; a.qscale = A.qscale;
    const int ns = A.nsplit;
    a.T = 16 * max(1, ((max(p, 0) + 15) / 16 + ns - 1) / ns);
    g = attn_geo_nk(a, c, p + 1);
    if (g.s == ns - 1 && g.t_s < p + 1) {
        g.t_e = p + 1;
        g.nsub = (g.t_e - g.t_s + 15) / 16;
    }
}

// ------------------------------------------------------------------ the kernel
__global__ void __launch_bounds__(NT) k_stream_decode(const Args* __restrict__ Ap) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const I4D_CONST Args& A = *(const I4D_CONST Args*)Ap;
    const int tid = i4d_tid();
    const int c = blockIdx.x, nwg = gridDim.x;
    float2* part = (float2*)(lds + OFF_PART);
    float* res = (float*)(lds + OFF_RES);
    float2* rope = (float2*)(lds + OFF_ROPE);
    KGeo* kg = (KGeo*)(lds + OFF_KG);
    SGeo* sg = (SGeo*)(lds + OFF_SG);
    float* red = (float*)(lds + OFF_RED);
    u32* sync = (u32*)(lds + OFF_SYNC);
    LPtr* tab = (LPtr*)(lds + OFF_TAB);
    const int D = A.D, F = A.F, qw = A.Hq * HD, kvw = A.Hkv * HD;

    // ---- set-up (all eight waves): layer table, position and RoPE table,
    // geometry, residual rows, sync words
    for (int i = tid; i < A.L * LPTR_WORDS; i += NT) ((u64*)tab)[i] = ld_g((const u64*)A.table + i);
    if (tid < 16) sync[tid] = 0u;
    int p = ld_g(A.pos);
    if (p < 0 || p > A.max_pos || p >= A.cap) {
        if (c == 0 && tid == 0) raise_status(A.status, I4D_DEV_BAD_POS);
        p = -1;
    }
    if (tid < HD / 2) {
        const double theta = pow(A.base, -2.0 * (double)tid / (double)HD);
        const double phi = (double)max(p, 0) * theta;
        double sn, cn;
        sincos(phi, &sn, &cn);
        rope[tid] = float2{(float)cn, (float)sn};
    }
    if (tid < 4) {
        KGeo k;
        const int kind = tid;
        int P, ci, nci, rows_half;
        k.K = kind == K_WO ? qw : kind == K_DN ? F : D;
        k.mat = 0; k.jump = 0u; k.jper = 0;
        if (kind == K_QKV) {
            k.mat = c < A.cq ? 0 : c < A.ck ? 1 : 2;
            P = (k.mat == 0 ? qw : kvw) / 2;
            ci = k.mat == 0 ? c : k.mat == 1 ? c - A.cq : c - A.ck;
            nci = k.mat == 0 ? A.cq : k.mat == 1 ? A.ck - A.cq : nwg - A.ck;
            k.mia = k.mib = k.mat;
        } else {
            P = kind == K_GU ? F : D / 2;
            ci = c; nci = nwg;
            k.mia = kind == K_WO ? 3 : kind == K_GU ? 4 : 6;
            k.mib = kind == K_GU ? 5 : k.mia;
        }
        k.S = k.K / 512;
        k.p0 = (int)(((long long)ci * P) / nci);
        k.np = (int)(((long long)(ci + 1) * P) / nci) - k.p0;
        k.U = k.np * k.S;
        k.n = (k.U + NSLOT - 1) / NSLOT;
        const unsigned rb = (unsigned)k.K / 2u, srb = (unsigned)k.K / 64u;
        if (kind == K_QKV) {
            const int row0 = (k.p0 / (HD / 2)) * HD + k.p0 % (HD / 2);
            k.ca_off = (unsigned)row0 * rb; k.cb_off = k.ca_off + (unsigned)(HD / 2) * rb;
            k.sa_off = (unsigned)row0 * srb; k.sb_off = k.sa_off + (unsigned)(HD / 2) * srb;
            k.jump = (unsigned)(HD / 2) * rb;
            k.jper = (HD / 2) * k.S;
        } else {
            rows_half = kind == K_GU ? 0 : D / 2;
            k.ca_off = (unsigned)k.p0 * rb; k.cb_off = (unsigned)(k.p0 + rows_half) * rb;
            k.sa_off = (unsigned)k.p0 * srb; k.sb_off = (unsigned)(k.p0 + rows_half) * srb;
        }
        kg[kind] = k;
    }
    __syncthreads();
    if (tid < 4 * NSLOT) {
        const int kind = tid / NSLOT, s = tid % NSLOT;
        const KGeo& k = kg[kind];
        SGeo g;
        g.u0 = (int)(((long long)s * k.U) / NSLOT);
        g.len = (int)(((long long)(s + 1) * k.U) / NSLOT) - g.u0;
        const int pl = k.S ? g.u0 / k.S : 0;
        g.seg0 = g.u0 - pl * k.S;
        g.pair0 = pl;
        const unsigned rb = (unsigned)k.K / 2u;
        int drow = pl;                                   // rows between pair p0's row a and this slot's first row a
        g.cnt0 = 1 << 30;
        if (kind == K_QKV) {
            const int pa = k.p0 + pl;
            drow = ((pa / (HD / 2)) * HD + pa % (HD / 2)) - ((k.p0 / (HD / 2)) * HD + k.p0 % (HD / 2));
            g.cnt0 = (HD / 2 - pa % (HD / 2)) * k.S - g.seg0;
        }
        g.off0 = (unsigned)drow * rb + (unsigned)g.seg0 * 256u;
        sg[tid] = g;
    }
    __syncthreads();
    // Per pair: the partial sums of the slots that met it, as indices into
    // part[slot][run] in slot order, so that an epilogue thread reads its
    // pair's few partials with independent loads.  Slot s touches pairs
    // pair0 .. pair0 + nr - 1 (run r is pair pair0 + r).
    {
        u32* pinfo = (u32*)(lds + OFF_PINFO);
        uint8_t* plist = (uint8_t*)(lds + OFF_PLIST);
        for (int i = tid; i < 4 * MAXNP; i += NT) {
            const int kind = i / MAXNP, pl = i % MAXNP;
            const KGeo& k = kg[kind];
            if (pl >= k.np) continue;
            int base = 0, cnt = 0;
#pragma unroll 4
            for (int s = 0; s < NSLOT; ++s) {
                const SGeo& q = sg[kind * NSLOT + s];
                const int nr = q.len > 0 ? (q.u0 + q.len - 1) / k.S - q.pair0 + 1 : 0;
                base += min(max(pl - q.pair0, 0), nr);              // entries of earlier pairs
                if (pl >= q.pair0 && pl < q.pair0 + nr) ++cnt;
            }
            pinfo[kind * MAXNP + pl] = ((u32)base << 8) | (u32)cnt;
            int e = base;
            for (int s = 0; s < NSLOT; ++s) {
                const SGeo& q = sg[kind * NSLOT + s];
                const int nr = q.len > 0 ? (q.u0 + q.len - 1) / k.S - q.pair0 + 1 : 0;
                if (pl >= q.pair0 && pl < q.pair0 + nr) plist[kind * NSLOT * MAXRUN + e++] = (uint8_t)(s * MAXRUN + (pl - q.pair0));
            }
        }
    }
    {   // residual rows of layer 0 (rows p and p + D/2 of this unit's Wo / W_down pairs)
        const KGeo& k = kg[K_WO];
        for (int i = tid; i < k.np; i += NT) {
            res[i] = ld_g(A.x_in + k.p0 + i);
            res[MAX_RES + i] = ld_g(A.x_in + k.p0 + i + D / 2);
        }
    }
    __syncthreads();

    // ---- the loader waves: the weight stream, and nothing else
    if (tid >= NCT) {
        loader_main(A, kg, sg, tab, lds + A.off_ring, sync, (tid >> 6) - NCW);
        return;
    }

    // ---- the consumer waves: every phase of every layer
    Spin sp{A.status, false};
    CBar cb{sync, A.status, 0u};
    const u32 tag = ld_g(A.epoch) + 1u;
    int t = 0, rslot = 0;                             // global step, its ring entry
    u32 rdy = 0u;                                     // steps the loader of this wave's half has written (last seen)
    AttnRegs<HD, ANSW> Rg;                            // K/V of the attention item's first round

    for (int ph = 0; ph < 4 * Ap->L; ++ph) {
        const I4D_CONST Args& A = *opaque_ptr(Ap);
        const int tid = i4d_tid(), lane = tid & 63, wave = tid >> 6, slot = tid >> 4, lane16 = tid & 15;
        const int kind = ph & 3, l = ph >> 2;
        const int D = A.D, F = A.F, G = A.Hq / A.Hkv, ps = A.ps;
        char* act = lds + A.off_act;                  // digit planes, then run scales (float)
        float* cs = (float*)(act + 4 * ps);
        // Exchange pointers of this layer, re-derived where used (see opaque_ptr)
#define I4D_RP(T, field) ((T*)(layer_region(Ap, l) + opaque_ptr(Ap)->field))

        if (kind == K_WO) {
            // ================= attention: item (KV head j, split s) of this unit
            const int items = A.Hkv * A.nsplit;
            if (c < items) {
                AttnArgs a;
                AttnGeo g;
                attn_setup(A, tab, l, c, p, a, g);
                const int ns = A.nsplit;
                // round 0 of the K/V loads went out during the q/k/v phase (Rg)
                u32x4* q32 = (u32x4*)(act + NCW * (16 * HD + 32) * 4);   // [HD / 32][2][64]
                uint16_t* knew = (uint16_t*)(act + ATT_LDS);
                uint16_t* vnew = knew + HD;
                const int r = lane & 15, gq = lane >> 4;
                static_assert(HD / 32 + 2 <= NCW, "one wave per 32-dim block of q, one each for the new k and v");
                if (wave < HD / 32) {
                    // q^T operand of head r of the group for the 16x16x32 instruction: wave mm
                    // takes 32-dim block mm, the 8 dims 32 mm + 8 gq .. + 7 as bf16 high and
                    // low parts (the blocks' exchange reads overlap instead of following each other)
                    const int mm = wave;
                    const u64* qrow = I4D_RP(u64, oq) + (size_t)(g.j * G + min(r, G - 1)) * HD + 8 * gq;
                    const float qs = (r < G) ? A.qscale : 0.f;
                    float t8[8];
                    ll_get<8>(qrow + 32 * mm, tag, t8, sp);
                    u32 hv[4], lv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float v0 = t8[2 * q] * qs, v1 = t8[2 * q + 1] * qs;
                        const uint16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
                        hv[q] = (u32)h0 | ((u32)h1 << 16);
                        lv[q] = (u32)f32_to_bf16(v0 - bf16_to_f32(h0)) | ((u32)f32_to_bf16(v1 - bf16_to_f32(h1)) << 16);
                    }
                    q32[(2 * mm) * 64 + lane] = u32x4{hv[0], hv[1], hv[2], hv[3]};
                    q32[(2 * mm + 1) * 64 + lane] = u32x4{lv[0], lv[1], lv[2], lv[3]};
                } else if (wave < HD / 32 + 2) {
                    const int kv = wave - HD / 32;              // 0: the new k, 1: the new v
                    float t2[2];
                    ll_get<2>(I4D_RP(u64, okv) + (size_t)g.j * 2 * HD + kv * HD + 2 * lane, tag, t2, sp);
                    uint16_t* dst = kv == 0 ? knew : vnew;
                    dst[2 * lane] = f32_to_bf16(t2[0]);          // the values are bf16 already: exact
                    dst[2 * lane + 1] = f32_to_bf16(t2[1]);
                }
                cbar(cb);
                const int stp = (g.kpos >= g.t_s && g.kpos < g.t_e) ? (g.kpos - g.t_s) / 16 : -1;
                float m = -INFINITY, lsum = 0.f;
                f4 O[HD / 16];
#pragma unroll
                for (int nt = 0; nt < HD / 16; ++nt) O[nt] = f4{0.f, 0.f, 0.f, 0.f};
                const int nround = (g.nsub + NCW * ANSW - 1) / (NCW * ANSW);
                for (int rnd = 0; rnd < nround; ++rnd) {
                    if (rnd > 0) {
                        // no load for a round whose only subtile of this wave is the new key alone
                        bool need = false;
#pragma unroll
                        for (int i = 0; i < ANSW; ++i) {
                            const int st = (rnd * ANSW + i) * NCW + wave;
                            need = need || (st < g.nsub && !(g.t_s + 16 * st == g.kpos && g.kpos == g.t_e - 1));
                        }
                        if (need) attn_load_round<HD, NCT, ANSW>(a, g, rnd, Rg);
                    }
#pragma unroll
                    for (int i = 0; i < ANSW; ++i) {
                        const int st = (rnd * ANSW + i) * NCW + wave;
                        if (st == stp) {
                            // the new key: its K row and V column from the exchange, not the cache
                            const int t0 = g.t_s + 16 * st;
                            if (t0 + r == g.kpos) {
#pragma unroll
                                for (int mm = 0; mm < HD / 32; ++mm) Rg.k[i][mm] = *(const u32x4*)(knew + 32 * mm + 8 * gq);
                            }
                            const int e = g.kpos - (t0 + 4 * gq);
                            if (e >= 0 && e < 4) {
#pragma unroll
                                for (int nt = 0; nt < HD / 16; ++nt) {
                                    const u32 nv = (u32)vnew[16 * nt + r];
                                    u32 lo = Rg.v[i][nt].x, hi = Rg.v[i][nt].y;
                                    if (e == 0) lo = (lo & 0xFFFF0000u) | nv;
                                    else if (e == 1) lo = (lo & 0x0000FFFFu) | (nv << 16);
                                    else if (e == 2) hi = (hi & 0xFFFF0000u) | nv;
                                    else hi = (hi & 0x0000FFFFu) | (nv << 16);
                                    Rg.v[i][nt] = u32x2{lo, hi};
                                }
                            }
                        }
                    }
                    // the round's subtiles two at a time (an odd last one with a masked partner)
#pragma unroll
                    for (int i = 0; i < ANSW; i += 2) {
                        const int st0 = (rnd * ANSW + i) * NCW + wave;
                        if (st0 >= g.nsub) continue;
                        if (i + 1 < ANSW)
                            attn_sub2<HD>(g, st0, st0 + NCW, Rg.k[i], Rg.v[i], Rg.k[i + 1], Rg.v[i + 1], q32, m, lsum, O);
                        else
                            attn_sub2<HD>(g, st0, g.nsub, Rg.k[i], Rg.v[i], Rg.k[i], Rg.v[i], q32, m, lsum, O);
                    }
                }
                attn_waves_to_lds<HD, NCT>(act, m, lsum, O);
                cbar(cb);
                const int hb = g.j * G;
                auto put = [&](int h, int d, float M, float Lv, float acc) {
                    u64* pr = I4D_RP(u64, opart) + ((size_t)(hb + h) * ns + g.s) * (HD + 2);
                    ll_put(pr + 2 + d, acc, tag);
                    if (d == 0) { ll_put(pr, M, tag); ll_put(pr + 1, Lv, tag); }
                };
                attn_combine_waves<HD, NCT>(act, G, put);
            }
            // ================= merge: head h, dims 32 qd .. 32 qd + 31 of this unit
            for (int it = c; it < A.Hq * 4; it += nwg) {
                const int h = it >> 2, qd = it & 3, ns = A.nsplit;
                cbar(cb);                                       // the attention's LDS is free again
                float* mv = (float*)act;                        // [ns]
                float* lv = mv + 64;                            // [ns]
                float* ov = lv + 64;                            // [ns][32]
                const u64* hp = I4D_RP(u64, opart) + (size_t)h * ns * (HD + 2);
                // one round: thread (s, q) fetches dims 2q, 2q + 1 of split s; threads of q = 0 also m and l
                for (int idx = tid; idx < ns * 16; idx += NCT) {
                    const int s = idx >> 4, q = idx & 15;
                    const u64* ps = hp + (size_t)s * (HD + 2);
                    // the split's (m, l) words are read together with its O words (one
                    // round trip); only a stale pair is fetched again
                    const u64x2 mlw = ld_g((const u64x2*)ps);
                    float t2[2];
                    ll_get<2>(ps + 2 + 32 * qd + 2 * q, tag, t2, sp);
                    ov[s * 32 + 2 * q] = t2[0];
                    ov[s * 32 + 2 * q + 1] = t2[1];
                    if (q == 0) {
                        float ml[2] = {__uint_as_float((u32)mlw.x), __uint_as_float((u32)mlw.y)};
                        if ((u32)(mlw.x >> 32) != tag || (u32)(mlw.y >> 32) != tag) ll_get<2>(ps, tag, ml, sp);
                        mv[s] = ml[0];
                        lv[s] = ml[1];
                    }
                }
                cbar(cb);
                if (tid < 32 * 8) {
                    // every wave: the largest running max over the splits (ns <= 64, one per lane)
                    float M = (lane < ns) ? mv[lane] : -INFINITY;
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
                    // thread (d, k): dim 32 qd + d, splits k, k + 8, ...; then a sum over the 8 k-lanes
                    const int d = tid >> 3, kk = tid & 7;
                    float acc = 0.f, Lsum = 0.f;
                    if (M != -INFINITY) {
                        for (int s = kk; s < ns; s += 8) {
                            const float w = exp2f(mv[s] - M);
                            acc = fmaf(ov[s * 32 + d], w, acc);
                            Lsum = fmaf(lv[s], w, Lsum);
                        }
                    }
#pragma unroll
                    for (int o = 4; o >= 1; o >>= 1) {
                        acc += __shfl_xor(acc, o);
                        Lsum += __shfl_xor(Lsum, o);
                    }
                    if (kk == 0)
                        pk_put((u32*)I4D_RP(u64, oo) + (size_t)h * HD + 32 * qd + d, Lsum > 0.f ? acc / Lsum : 0.f, tag);
                }
            }
            cbar(cb);                                           // before the staging reuses the LDS
        }

        // ================= stage this phase's activations (digits in LDS)
        const KGeo& k = kg[kind];
        {
            const int K = k.K, ngr = K / 8;
            // six digit planes (23 bits) for the k and v rows, which are rounded to
            // bf16 into the cache; four (15 bits) for q, which attention splits into
            // bf16 high and low parts (16 bits) anyway, and for the other phases
            const bool six = kind == K_QKV && kg[K_QKV].mat != 0;
            // normalised inputs (x, y: K = D <= 8192, RMN rounds of groups): RMSNorm, then digits
            // the gain words of this thread's groups, loaded before the exchange
            // fetch so that their latency hides under it
            auto load_gain = [&](const uint16_t* gain, u32x4 (&gw)[RMN]) {
#pragma unroll
                for (int rr = 0; rr < RMN; ++rr) gw[rr] = ld_g((const u32x4*)(gain + 8 * min(rr * NCT + tid, ngr - 1)));
            };
            // RMSNorm's 1/rms is one factor per token, so it multiplies the
            // pair sums in the epilogue instead: the digits are those of
            // gain * x (each run takes its own power of two, so the scale of
            // the run does not matter), and the sum of squares needs no
            // barrier of its own -- each wave leaves its share in red[] before
            // the barrier that ends the staging
            auto norm_stage = [&](float (&v)[RMN][8], const u32x4 (&gw)[RMN]) {
                float ss = 0.f;
#pragma unroll
                for (int rr = 0; rr < RMN; ++rr)
                    if (rr * NCT + tid < ngr)
#pragma unroll
                        for (int e = 0; e < 8; ++e) ss = fmaf(v[rr][e], v[rr][e], ss);
#pragma unroll
                for (int rr = 0; rr < RMN; ++rr) {
                    const int g = rr * NCT + tid;
                    if (g < ngr) {
                        const u32 gws[4] = {gw[rr].x, gw[rr].y, gw[rr].z, gw[rr].w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            v[rr][e] *= __uint_as_float((e & 1) ? (gws[e >> 1] & 0xFFFF0000u) : (gws[e >> 1] << 16));
                        digitize8(act, ps, cs, g, v[rr], six, A.status);
                    }
                }
                wave_share(ss, red);
            };
            if (kind == K_QKV) {
                float v[RMN][8];
                u32x4 gw[RMN];
                load_gain(tab[l].g1, gw);
                if (l == 0) {                                  // the caller's fp32 input
#pragma unroll
                    for (int rr = 0; rr < RMN; ++rr) {
                        const int g = min(rr * NCT + tid, ngr - 1);
                        const f4 a0 = ld_g((const f4*)(A.x_in + 8 * g)), a1 = ld_g((const f4*)(A.x_in + 8 * g + 4));
                        v[rr][0] = a0.x; v[rr][1] = a0.y; v[rr][2] = a0.z; v[rr][3] = a0.w;
                        v[rr][4] = a1.x; v[rr][5] = a1.y; v[rr][6] = a1.z; v[rr][7] = a1.w;
                    }
                } else {
                    fetch_groups<RMN, true>(I4D_RP(u64, ox), 0, ngr, tag, v, sp);
                }
                norm_stage(v, gw);
            } else if (kind == K_GU) {
                float v[RMN][8];
                u32x4 gw[RMN];
                load_gain(tab[l].g2, gw);
                fetch_groups<RMN, false>(I4D_RP(u64, oy), 0, ngr, tag, v, sp);
                norm_stage(v, gw);
            } else if (kind == K_WO) {
                float v[RMN][8];                               // q width <= 8192
                fetch_groups<RMN, false>(I4D_RP(u64, oo), 0, ngr, tag, v, sp);
#pragma unroll
                for (int rr = 0; rr < RMN; ++rr)
                    if (rr * NCT + tid < ngr) digitize8(act, ps, cs, rr * NCT + tid, v[rr], false, A.status);
            } else {
                for (int g0 = 0; g0 < ngr; g0 += RMD * NCT) {  // d_ff <= 32768: passes of RMD rounds
                    float v[RMD][8];
                    fetch_groups<RMD, false>(I4D_RP(u64, oact), g0, ngr, tag, v, sp);
#pragma unroll
                    for (int rr = 0; rr < RMD; ++rr)
                        if (g0 + rr * NCT + tid < ngr) digitize8(act, ps, cs, g0 + rr * NCT + tid, v[rr], false, A.status);
                }
            }
        }
        cbar(cb);
        if (kind == K_QKV && c < A.Hkv * A.nsplit) {
            // The cached keys of this layer's attention item do not depend on this
            // step: their first round of loads goes out now and lands while the
            // weights stream (the staging above had to wait for its exchange
            // loads alone; nothing waits on vector memory until the attention).
            AttnArgs a;
            AttnGeo g;
            attn_setup(A, tab, l, c, p, a, g);
            attn_load_round<HD, NCT, ANSW>(a, g, 0, Rg);
        }

        // ================= this phase's weight units, from the ring
        {
            const int n = uni(k.n), S = k.S;
            const SGeo& s = sg[kind * NSLOT + slot];
            const int len = s.len;
            int seg = s.seg0, run = 0;
            unsigned aoff = (unsigned)seg * 256u + (unsigned)lane16 * 16u;
            const int hs = ((lane16 >> 2) & 1) ? 0 : 16;
            const bool six = kind == K_QKV && k.mat != 0;
            // this wave's place in the ring: its loader's half, its 2 KB of codes, its slots' scale words
            const int lw = wave / CPL, cw = wave - CPL * lw;
            const char* half = lds + A.off_ring + (size_t)lw * A.nb * HSTEP;
            const unsigned uoff = (unsigned)(cw * 2048 + lane * 16);
            const unsigned soff = (unsigned)(CPL * 2048 + (4 * (4 * cw + (lane >> 4)) + (lane16 >> 3)) * 4);
            const u32* ready = sync + SY_READY + lw;
            u32* cons = sync + SY_CONS + wave;
            const int nb = A.nb;
            float ra = 0.f, rb = 0.f;
            for (int j = 0; j < n; ++j) {
                if ((int)rdy < t + 1) rdy = lds_wait([&] { return lds_get(ready); }, (u32)(t + 1), sync, A.status);
                if (j < len) {
                    const char* e = half + rslot * HSTEP;
                    Unit u;
                    u.a = *(const u32x4*)(e + uoff);
                    u.b = *(const u32x4*)(e + uoff + 1024);
                    u.sa = *(const u32*)(e + soff);
                    u.sb = *(const u32*)(e + soff + 8);
                    dot_unit(u, act, ps, aoff, cs[aoff >> 4], hs, six, ra, rb);
                    ++seg;
                    aoff += 256u;
                    const bool wrap = seg == S;
                    if (wrap || j == len - 1) {
                        const float va = row16_sum(ra), vb = row16_sum(rb);
                        if (lane16 == 0 && run < MAXRUN) part[slot * MAXRUN + run] = float2{va, vb};
                        ++run;
                        ra = 0.f; rb = 0.f;
                    }
                    if (wrap) { seg = 0; aoff = (unsigned)lane16 * 16u; }
                }
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                if (lane == 0) lds_put(cons, (u32)(t + 1));  // after this wave's reads of entry rslot
                ++t;
                rslot = rslot + 1 == nb ? 0 : rslot + 1;
            }
        }
        cbar(cb);

        // ================= per-pair totals (fixed slot order) and the phase's epilogue
        // One thread per pair (np < NCT: see below).
        static_assert(MAXNP < NCT, "runs_of() <= MAXRUN bounds the pairs per unit below NCT");
        if (tid < k.np) {
            const int pl = tid;
            float va = 0.f, vb = 0.f;
            {   // the partials of the slots that met this pair, in slot order
                const u32 pi = ((const u32*)(lds + OFF_PINFO))[kind * MAXNP + pl];
                const uint8_t* pe = (const uint8_t*)(lds + OFF_PLIST) + kind * NSLOT * MAXRUN + (pi >> 8);
                const int cnt = (int)(pi & 255u);
#pragma unroll 4
                for (int e = 0; e < cnt; ++e) {
                    const float2 t = part[pe[e]];
                    va += t.x;
                    vb += t.y;
                }
            }
            const int pm = k.p0 + pl;                          // pair index within its matrix
            if (kind == K_QKV || kind == K_GU) {               // RMSNorm's 1/rms (see the staging)
                float ssq = 0.f;
#pragma unroll
                for (int w = 0; w < NCW; ++w) ssq += red[w];
                const float rs = 1.0f / sqrtf(ssq / (float)k.K + A.eps);
                va *= rs;
                vb *= rs;
            }
            if (kind == K_QKV) {
                const int head = pm / (HD / 2), i = pm % (HD / 2);
                float xa = va, xb = vb;
                if (k.mat < 2) {
                    const float2 rc = rope[i];
                    xa = va * rc.x - vb * rc.y;
                    xb = va * rc.y + vb * rc.x;
                }
                if (k.mat == 0) {
                    ll_put(I4D_RP(u64, oq) + (size_t)head * HD + i, xa, tag);
                    ll_put(I4D_RP(u64, oq) + (size_t)head * HD + i + HD / 2, xb, tag);
                } else {
                    const uint16_t ba = f32_to_bf16(xa), bb = f32_to_bf16(xb);
                    u64* nr = I4D_RP(u64, okv) + (size_t)head * 2 * HD + (k.mat - 1) * HD;
                    ll_put(nr + i, bf16_to_f32(ba), tag);
                    ll_put(nr + i + HD / 2, bf16_to_f32(bb), tag);
                    if (p >= 0) {
                        const size_t tile = ((size_t)head * A.cap + (size_t)(p >> 4) * 16) * HD;
                        const int tp = p & 15;
                        if (k.mat == 1) {
                            uint16_t* kt = tab[l].kc + tile;
                            st_g(kt + (i >> 5) * 512 + tp * 32 + (i & 31), ba);
                            st_g(kt + ((i + HD / 2) >> 5) * 512 + tp * 32 + ((i + HD / 2) & 31), bb);
                        } else {
                            uint16_t* vt = tab[l].vc + tile;
                            st_g(vt + (size_t)i * 16 + tp, ba);
                            st_g(vt + (size_t)(i + HD / 2) * 16 + tp, bb);
                        }
                    }
                }
            } else if (kind == K_WO) {
                const float ya = res[pl] + va, yb = res[MAX_RES + pl] + vb;
                res[2 * MAX_RES + pl] = ya;
                res[3 * MAX_RES + pl] = yb;
                pk_put((u32*)I4D_RP(u64, oy) + pm, ya, tag);
                pk_put((u32*)I4D_RP(u64, oy) + pm + D / 2, yb, tag);
            } else if (kind == K_GU) {
                pk_put((u32*)I4D_RP(u64, oact) + pm, va / (1.0f + expf(-va)) * vb, tag);
            } else {
                const float za = res[2 * MAX_RES + pl] + va, zb = res[3 * MAX_RES + pl] + vb;
                res[pl] = za;
                res[MAX_RES + pl] = zb;
                if (l + 1 == A.L) {
                    st_g(A.x_out + pm, za);
                    st_g(A.x_out + pm + D / 2, zb);
                } else {
                    u64* xn = (u64*)(A.lbase + (size_t)(l + 1) * A.lstride + A.ox);
                    ll_put(xn + pm, za, tag);
                    ll_put(xn + pm + D / 2, zb, tag);
                }
            }
        }
        // No barrier here: the next writes of part[] (the next stream) and of
        // the staging area come after the next phase's staging barrier, which
        // every wave reaches only after its epilogue; res[] rows are read and
        // written by the same thread.
    }
#undef I4D_RP
    wait_stores();
    // every workgroup read the epoch before any of them could finish (each
    // waits for data from all others), so the next launch's epoch goes out now
    if (blockIdx.x == 0 && i4d_tid() == 0) st_dev_t(opaque_ptr(Ap)->epoch, tag);
}

// The launch arguments, passed by value, into the workspace (the kernel reads
// them through a pointer, re-reading fields where they are used).
// One word per thread: every read of the argument is issued at once.
constexpr int FILL_NT = 512;
static_assert(sizeof(Args) % 8 == 0 && sizeof(Args) / 8 <= FILL_NT, "one word of Args per thread");
__global__ void __launch_bounds__(FILL_NT) k_fill_args(Args a, Args* dst) {
    constexpr int W = (int)(sizeof(Args) / 8);
    const int i = i4d_tid();
    if (i < W) ((u64*)dst)[i] = ((const u64*)&a)[i];
}

// Copy a chunk of layer-table entries (passed by value) into the workspace.
constexpr int LPTR_PER_FILL = 24;
static_assert(LPTR_PER_FILL * LPTR_WORDS <= FILL_NT, "one table word per thread");
struct LPtrChunk { LPtr e[LPTR_PER_FILL]; LPtr* dst; int count; };
__global__ void __launch_bounds__(FILL_NT) k_fill_ltab(LPtrChunk ch) {
    const int i = i4d_tid();
    if (i < ch.count * LPTR_WORDS) ((u64*)ch.dst)[i] = ((const u64*)ch.e)[i];
}

// ------------------------------------------------------------------ host side
inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Region {
    size_t args, table, zero, layer0, lstride;
    size_t ox, oq, okv, opart, oo, oy, oact;
    size_t total;
};

// Key-axis splits per KV head: one attention item per compute unit, at most
// 64 (the merge stages one head's partials of every split in LDS).
int splits_of(const i4d_config* c, int nwg) { return std::max(1, std::min(64, nwg / c->n_kv_heads)); }

Region region_of(const i4d_config* c, int n_layers, int nwg) {
    Region r;
    size_t off = 0;
    r.args = off; off = a256(off + sizeof(Args));
    r.table = off; off = a256(off + (size_t)MAX_LAYERS * sizeof(LPtr));
    r.zero = off; off = a256(off + 1024);
    r.layer0 = off;
    const size_t D = c->d_model, F = c->d_ff, qw = (size_t)c->n_q_heads * HD, kvw = (size_t)c->n_kv_heads * HD;
    const size_t ns = splits_of(c, nwg);
    size_t lo = 0;
    auto take = [&](size_t words) { const size_t o = lo; lo = a256(lo + words * 8); return o; };
    r.ox = take(D);
    r.oq = take(qw);
    r.okv = take(2 * kvw);
    r.opart = take((size_t)c->n_q_heads * ns * (HD + 2));
    r.oo = take(qw);
    r.oy = take(D);
    r.oact = take(F);
    r.lstride = lo;
    r.total = off + (size_t)n_layers * lo;
    return r;
}

}  // namespace

size_t region_bytes(const i4d_config* c, int n_layers, int nwg) { return region_of(c, n_layers, nwg).total; }

namespace {

// Every host-side decision of one launch, taken before anything is enqueued.
struct Plan {
    int cq, ck;          // q/k/v split of the compute units
    int ps, nb;          // LDS bytes per digit plane; ring steps
    unsigned off_act, off_ring;
    size_t lds;
};

constexpr int LDS_MAX = 160 * 1024;

// LDS of one launch: the fixed part and the layer table, the staging area
// (four digit planes of ps bytes and the run scales, or attention's working
// set), then as many ring steps as fit (at most NBMAX).
void lds_plan(const i4d_config* c, int n_layers, Plan& P) {
    const int D = c->d_model, F = c->d_ff, qw = c->n_q_heads * HD;
    const int kmax = std::max(D, std::max(qw, F));
    P.ps = (int)a256((size_t)std::max(kmax / 2, D));        // six planes for q/k/v need d_model <= ps
    const size_t stage = (size_t)4 * P.ps + (size_t)P.ps / 4;
    const size_t att = (size_t)ATT_LDS + 2 * HD * 2;
    P.off_act = (unsigned)a256((size_t)OFF_TAB + (size_t)n_layers * sizeof(LPtr));
    P.off_ring = P.off_act + (unsigned)a256(std::max(stage, std::max(att, (size_t)MERGE_LDS)));
    const long room = (long)LDS_MAX - (long)P.off_ring;
    P.nb = room > 0 ? (int)std::min<long>(NBMAX, room / (NLW * HSTEP)) : 0;
    P.lds = (size_t)P.off_ring + (size_t)NLW * std::max(P.nb, 0) * HSTEP;
}

// q/k/v rows go to compute units in proportion: [0, cq) q, [cq, ck) k, [ck, nwg) v.
void qkv_split(const i4d_config* c, int nwg, int& cq, int& ck) {
    const int npq = c->n_q_heads * HD / 2, npk = c->n_kv_heads * HD / 2;
    // q rows cost about 10 units per step, k and v rows 14 (six digit planes against four)
    int nq = (int)((long long)nwg * npq * 10 / (npq * 10 + 2 * npk * 14));
    nq = std::min(std::max(nq, 1), nwg - 2);
    const int nk = std::max(1, (nwg - nq) / 2);
    cq = nq;
    ck = nq + nk;
}

// Runs per slot of a phase whose compute unit holds np pairs of S units.
int runs_of(int np, int S) {
    const int n = (np * S + NSLOT - 1) / NSLOT;
    return (n + S - 1) / S + 1;
}

bool make_plan(const i4d_config* c, int n_layers, const i4d_layer* layers, const i4d_kv* kv, int batch, int nwg, Plan& P) {
    if (batch != 1 || c->head_dim != HD || n_layers < 1 || n_layers > MAX_LAYERS) return false;
    const int D = c->d_model, F = c->d_ff, qw = c->n_q_heads * HD, kvw = c->n_kv_heads * HD;
    if (c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads) return false;
    if (c->n_q_heads / c->n_kv_heads > 16) return false;
    // every K a whole number of 512-input units and within one digit plane;
    // D and the q width at most two staging rounds of the workgroup
    if (D % 512 || F % 512 || qw % 512 || F > KMAX || D > 8192 || qw > 8192) return false;
    static_assert(RMN * NCT * 8 >= 8192, "d_model and the q width within RMN staging rounds");
    if (nwg < 3 || nwg > 1024) return false;
    if ((D / 2 + nwg - 1) / nwg > MAX_RES) return false;     // residual rows per compute unit
    for (int l = 0; l < n_layers; ++l) {
        const i4d_layer& L = layers[l];
        const i4d_mat* m[7] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
        for (int i = 0; i < 7; ++i) {
            if (m[i]->dtype != I4D_WEIGHT_INT4 || m[i]->group != 128) return false;
            if (((uintptr_t)m[i]->data % 16) || ((uintptr_t)m[i]->scales % 4)) return false;
        }
        if (kv[l].pages || kv[l].capacity != kv[0].capacity) return false;
        if (((uintptr_t)L.attn_norm % 16) || ((uintptr_t)L.ffn_norm % 16)) return false;
    }
    // pair runs per slot within MAXRUN in every phase
    qkv_split(c, nwg, P.cq, P.ck);
    const int nq = P.cq, nk = P.ck - P.cq, nv = nwg - P.ck;
    if (nk < 1 || nv < 1) return false;
    const int pqkv = std::max((qw / 2 + nq - 1) / nq, std::max((kvw / 2 + nk - 1) / nk, (kvw / 2 + nv - 1) / nv));
    if (runs_of(pqkv, D / 512) > MAXRUN) return false;
    if (runs_of((D / 2 + nwg - 1) / nwg, qw / 512) > MAXRUN) return false;
    if (runs_of((F + nwg - 1) / nwg, D / 512) > MAXRUN) return false;
    if (runs_of((D / 2 + nwg - 1) / nwg, F / 512) > MAXRUN) return false;
    // LDS, no scratch, one workgroup per compute unit
    lds_plan(c, n_layers, P);
    if (P.nb < 2 || P.lds > (size_t)LDS_MAX) return false;
    static int lds_set[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    if (lds_set[dev] < (int)P.lds) {
        if (hipFuncSetAttribute((const void*)k_stream_decode, hipFuncAttributeMaxDynamicSharedMemorySize, (int)P.lds) != hipSuccess)
            return false;
        lds_set[dev] = (int)P.lds;
    }
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, (const void*)k_stream_decode) != hipSuccess || fa.localSizeBytes != 0) return false;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_stream_decode, NT, P.lds) != hipSuccess) return false;
    return per_cu >= 1;
}

}  // namespace

bool supported(const i4d_config* c, int n_layers, const i4d_layer* layers, const i4d_kv* kv, int batch, int nwg) {
    Plan P;
    return make_plan(c, n_layers, layers, kv, batch, nwg, P);
}

int run(const i4d_config* c, int n_layers, const i4d_layer* layers, const float* x_in, float* x_out, const i4d_kv* kv,
        const int* pos, int max_pos, char* region, int* status, unsigned* epoch, int nwg, hipStream_t s,
        hipEvent_t* timing_ev) {
    Plan P;
    if (!make_plan(c, n_layers, layers, kv, 1, nwg, P)) return I4D_EUNSUPPORTED;
    hipStreamCaptureStatus cap_st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap_st) != hipSuccess) return I4D_EHIP;
    const Region R = region_of(c, n_layers, nwg);

    LPtr* table = (LPtr*)(region + R.table);
    for (int l0 = 0; l0 < n_layers; l0 += LPTR_PER_FILL) {
        LPtrChunk ch;
        memset(&ch, 0, sizeof(ch));
        ch.count = std::min(LPTR_PER_FILL, n_layers - l0);
        ch.dst = table + l0;
        for (int i = 0; i < ch.count; ++i) {
            const i4d_layer& Ls = layers[l0 + i];
            const i4d_mat* m[7] = {&Ls.wq, &Ls.wk, &Ls.wv, &Ls.wo, &Ls.wg, &Ls.wu, &Ls.wd};
            LPtr& d = ch.e[i];
            for (int k = 0; k < 7; ++k) { d.c[k] = (const uint8_t*)m[k]->data; d.s[k] = (const uint8_t*)m[k]->scales; }
            d.g1 = Ls.attn_norm;
            d.g2 = Ls.ffn_norm;
            d.kc = kv[l0 + i].k;
            d.vc = kv[l0 + i].v;
        }
        hipLaunchKernelGGL(k_fill_ltab, dim3(1), dim3(FILL_NT), 0, s, ch);
    }

    Args A;
    memset(&A, 0, sizeof(A));
    A.table = table;
    A.L = n_layers;
    A.x_in = x_in;
    A.x_out = x_out;
    A.pos = pos;
    A.max_pos = max_pos;
    A.cap = kv[0].capacity;
    A.D = c->d_model; A.F = c->d_ff; A.Hq = c->n_q_heads; A.Hkv = c->n_kv_heads;
    A.eps = c->rms_eps;
    A.qscale = (float)(1.4426950408889634 / sqrt((double)HD));
    A.base = c->rope_base;
    A.nsplit = splits_of(c, nwg);
    A.cq = P.cq; A.ck = P.ck;
    A.ps = P.ps; A.nb = P.nb;
    A.off_act = P.off_act; A.off_ring = P.off_ring;
    A.lbase = region + R.layer0;
    A.lstride = R.lstride;
    A.ox = (unsigned)R.ox; A.oq = (unsigned)R.oq; A.okv = (unsigned)R.okv; A.opart = (unsigned)R.opart;
    A.oo = (unsigned)R.oo; A.oy = (unsigned)R.oy; A.oact = (unsigned)R.oact;
    A.zero = (const uint8_t*)(region + R.zero);
    A.status = status;
    A.epoch = epoch;
    hipLaunchKernelGGL(k_fill_args, dim3(1), dim3(FILL_NT), 0, s, A, (Args*)(region + R.args));

    if (timing_ev) (void)hipEventRecord(timing_ev[0], s);
    hipError_t e;
    const Args* Ad = (const Args*)(region + R.args);
    if (cap_st == hipStreamCaptureStatusNone) {
        void* args[] = {&Ad};
        e = hipLaunchCooperativeKernel((const void*)k_stream_decode, dim3(nwg), dim3(NT), args, (unsigned)P.lds, s);
    } else {
        // inside a graph capture: an ordinary launch of one workgroup per compute
        // unit (a graph replays its kernels one after another, so every workgroup
        // is resident; a workgroup that waits too long gives up, never hangs)
        hipLaunchKernelGGL(k_stream_decode, dim3(nwg), dim3(NT), P.lds, s, Ad);
        e = hipGetLastError();
    }
    if (timing_ev) (void)hipEventRecord(timing_ev[1], s);
    return e == hipSuccess ? I4D_OK : I4D_EHIP;
}

}  // namespace i4d_stream
