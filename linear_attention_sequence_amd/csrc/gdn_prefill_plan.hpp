// Index arithmetic of the MFMA prefill (d_k = d_v = 128, chunks of C = 64 tokens): the
// workspace layout, how a prompt's chunks split into carry segments, the blockIdx maps
// of the chunk and carry kernels, the regions of a carry LDS stage and the row and
// 16-byte granule each lane loads into them. The kernels compute every address from
// these functions, and so does the host-side bounds model of the carry
// (tests/carry_model.cpp), so the model checks the arithmetic the GPU runs.
//
// Everything here is constexpr (usable from host and device code alike) or plain host
// code, with no HIP types.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace gdn {
namespace plan {

constexpr int C = 64;       // chunk length
constexpr int D = 128;      // head dim (dk == dv)
// per (chunk, V head) coefficients: [0, C) exp(Gam_t); [C, 2C) exp(Gam_last - Gam_t);
// 2C: exp(Gam_last); 2C + 1: 2^uexp, the scale of the stored U; padded to 40 granules
constexpr int COEF = 160;

// Contraction order of the carry's A operands. Its B operands are accumulator tiles
// (a lane holds rows 4 g .. 4 g + 3 of every 16-row tile), so the eight k slots of
// lane group g in step ks are the logical indices 32 ks + 4 g + (0..3) and
// 32 ks + 16 + 4 g + (0..3). Operands contracted over the state's rows (W, q_hat, the
// key features) and over tokens (K^T, P) are stored in that order, so that a lane's
// eight halfs are one 16-byte read: logical index k = 32 b + 16 h + 4 g + e sits at
// position kpos(k) = 32 b + 8 g + 4 h + e, and position p holds kidx(p).
constexpr int kpos(int k) {
    return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}
constexpr int kidx(int p) {
    return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}
static_assert(kidx(kpos(45)) == 45 && kpos(kidx(45)) == 45 && kpos(16) == 4 && kpos(4) == 8, "k order");

constexpr int imin(int a, int b) { return a < b ? a : b; }
constexpr long long lmin(long long a, long long b) { return a < b ? a : b; }

// ---- raw value loads of the chunk kernel --------------------------------------------
// A chunk (not a sequence's first) whose C tokens are all present takes its values' 12 raw
// positions per item in two vector loads, from p - 4 + par (p = the item's first token, par
// = the parity of the item's element offset ch L + p - 4 inside the row, so that the loads
// start on a 4-byte boundary); the loads then reach position pc + C - 1 + par of the
// channel's row. With an even row length L the parity is that of the chunk's first
// position pc for every channel; with an odd one it can be either.
constexpr int value_load_parity_max(int L, int pc) { return (L & 1) != 0 ? 1 : (pc & 1); }
constexpr bool value_fast(int c, int nt, int pc, int L) {
    return c > 0 && nt == C && pc + C + value_load_parity_max(L, pc) <= L;
}
// ---- segments of the carry ---------------------------------------------------------
// Unpacked prompts whose heads leave the CUs idle run the carry in segments. Its second
// pass runs 2 (nseg - 1) half-head workgroups per head (nseg - 1 whole-head ones when
// the gated RMSNorm is fused into the output store: `whole`), sized to about one round
// of the CUs, and its first 2 nseg - 3 whole-head ones; a segment averages at least
// kMinSegChunks chunks, and nseg >= 3 (with two segments the two passes are one chain
// cut in two). With `whole` the first pass may take two rounds: at L = 4096 eight
// segments (first pass 416 workgroups, second 224) beat five (224 and 128) by 4 us.
constexpr int kMaxSeg = 8;
constexpr int kMinSegChunks = 4;
constexpr int kLayoutCUs = 256;   // the workspace is sized for this many CUs at most
// Segment 0 alone also forms its outputs in the first pass, at whole-head speed, so it
// gets kSeg0 / 8 of the share of each other segment.
constexpr int kSeg0 = 5;

constexpr int chunks_of_len(int len) { return (len + C - 1) / C; }

constexpr int max_chunks(int B, int L, int N, bool ragged) {
    return ragged ? chunks_of_len(L) + N : B * chunks_of_len(L);
}

constexpr int segments(int B, int L, int N, int Hv, bool ragged, int cus, bool whole = false) {
    if (ragged || B != N || N <= 0 || Hv <= 0) return 1;
    const long long heads = static_cast<long long>(N) * Hv;
    long long ks = cus / ((whole ? 1 : 2) * heads) + 1;
    ks = lmin(ks, kMaxSeg);
    ks = lmin(ks, chunks_of_len(L) / kMinSegChunks);
    return ks >= 3 ? static_cast<int>(ks) : 1;
}

// First chunk of segment j (0 <= j <= nseg) of a sequence of nch chunks; seg0 is segment
// 0's weight in eighths (the bounds model sweeps it; the kernels use kSeg0).
constexpr int seg_begin(int nch, int nseg, int j, int seg0 = kSeg0) {
    if (j <= 0) return 0;
    if (j >= nseg) return nch;
    const int den = seg0 + 8 * (nseg - 1);
    return (nch * (seg0 + 8 * (j - 1)) + den / 2) / den;
}

// ---- workspace -------------------------------------------------------------------
constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Byte offsets of the workspace regions (from a 256-byte aligned base) and their sizes
// in elements of their types.
struct Layout {
    size_t qh, kh, W, U, P, KT, coef, cbase, Sent, Mhl, Mexp, Rseg, bytes;
    size_t n_qh, n_kh, n_W, n_U, n_P, n_KT, n_coef, n_cbase, n_Sent, n_Mhl, n_Mexp, n_Rseg;
    int nc_max, nseg;
};

// `whole`: the layout of a call with the gated RMSNorm fused (its own segment count).
constexpr Layout layout(int B, int L, int N, int Hk, int Hv, bool ragged, bool whole) {
    Layout w{};
    const size_t T = static_cast<size_t>(B) * L;
    const size_t nc = static_cast<size_t>(max_chunks(B, L, N, ragged));
    size_t off = 0;
    w.n_qh = T * Hk * D;       w.qh = off;   off = align256(off + w.n_qh * 2);
    w.n_kh = T * Hk * D;       w.kh = off;   off = align256(off + w.n_kh * 2);
    w.n_W = nc * Hv * C * D;   w.W = off;    off = align256(off + w.n_W * 2);
    w.n_U = nc * Hv * C * D;   w.U = off;    off = align256(off + w.n_U * 2);
    w.n_P = nc * Hv * C * C;   w.P = off;    off = align256(off + w.n_P * 2);
    w.n_KT = nc * Hk * D * C;  w.KT = off;   off = align256(off + w.n_KT * 2);
    w.n_coef = nc * Hv * COEF; w.coef = off; off = align256(off + w.n_coef * 4);
    if (ragged) {              // packed prompts: each sequence's first chunk slot, and the total
        w.n_cbase = static_cast<size_t>(N) + 1; w.cbase = off; off = align256(off + w.n_cbase * 4);
    }
    w.nseg = segments(B, L, N, Hv, ragged, kLayoutCUs, whole);
    if (w.nseg > 1) {
        const size_t tiles = static_cast<size_t>(N) * Hv * D * D;
        const size_t mid = static_cast<size_t>(w.nseg - 2);
        w.n_Sent = tiles;                 w.Sent = off; off = align256(off + w.n_Sent * 4);
        w.n_Mhl = mid * tiles * 2;        w.Mhl = off;  off = align256(off + w.n_Mhl * 2);
        w.n_Mexp = mid * N * Hv * (D / 16); w.Mexp = off; off = align256(off + w.n_Mexp * 4);
        w.n_Rseg = mid * tiles;           w.Rseg = off; off = align256(off + w.n_Rseg * 4);
    }
    w.nc_max = static_cast<int>(nc);
    w.bytes = off;
    return w;
}

// ---- chunk kernel: blockIdx -> (chunk id, V head) ------------------------------------
// The f V heads of a K head read the same keys and queries: they are dispatched 8
// blockIdx apart, i.e. to one XCD, whose L2 then serves the second read; the tail that
// does not fill a group of 8 (chunk, K head) units is laid out unit-major.
struct ChunkUnit { int id, hk, h; };
constexpr ChunkUnit chunk_unit(int block, int nc_max, int Hk, int Hv) {
    const int f = Hv / Hk;
    const int units = nc_max * Hk, grp = units / 8, full = 8 * f * grp;
    int u = 0, hl = 0;
    if (block < full) {
        u = (block / (8 * f)) * 8 + block % 8;
        hl = (block / 8) % f;
    } else {
        const int rem = block - full, tail = units - 8 * grp;
        u = 8 * grp + rem % tail;
        hl = rem / tail;
    }
    const int hk = u % Hk;
    return ChunkUnit{u / Hk, hk, hk * f + hl};
}

// ---- carry kernel ----------------------------------------------------------------
// kinds of workgroup per head: 1 unsegmented; pass 1: FIRST + (LOCAL, XMAP) per middle
// segment; pass 2: one per segment 1 .. nseg - 1
constexpr int carry_kinds(int nseg, int pass) {
    return nseg <= 1 ? 1 : (pass == 1 ? 2 * nseg - 3 : nseg - 1);
}

// blockIdx -> (slice, slot): the nsl = kinds * (workgroups per head) slices of a slot
// (sequence, head) are dispatched together and 8 blockIdx apart, i.e. on one XCD,
// sharing its L2 for the operands they read; the tail that does not fill a group of 8
// slots is laid out slice-major.
struct Slice { int slice, slot; };
constexpr Slice carry_slice(int block, int nsl, int nh) {
    if (nsl <= 1) return Slice{0, block};
    const int grp = nh / 8, full = 8 * nsl * grp;
    if (block < full) {
        const int w = block % (8 * nsl);
        return Slice{w / 8, (block / (8 * nsl)) * 8 + w % 8};
    }
    const int rem = block - full, tail = nh - 8 * grp;
    return Slice{rem / tail, 8 * grp + rem % tail};
}

// blockIdx -> (slice, sequence slot, V head) of the carry: the f = Hv / Hk V heads that
// share a K head form one dispatch unit of f * nsl slices (carry_slice over (sequence,
// K head) units), so every workgroup that reads a chunk's keys and queries runs on one XCD.
struct CarryUnit { int slice, n, h; };
constexpr CarryUnit carry_unit(int block, int nsl, int N, int Hk, int Hv) {
    const int f = Hv / Hk;
    const Slice s = carry_slice(block, nsl * f, N * Hk);
    return CarryUnit{s.slice % nsl, s.slot / Hk, (s.slot % Hk) * f + s.slice / nsl};
}

// What a carry workgroup of a given kind does: segment sj, its entry state, whether it
// forms outputs and loads U, and where its end state goes.
enum Entry { kFromState = 0, kFromZero = 1, kFromIdentity = 2 };
enum EndTo { kEndS = 0, kEndSent = 1, kEndRseg = 2, kEndNone = 3 };
struct Job {
    int sj;        // segment
    int entry;     // Entry: the state it starts from (pass 2: S_1 or a later R, see below)
    bool outs;     // forms outputs (reads q_hat and P)
    bool useU;     // reads U (U = 0 for the identity carry)
    int end;       // EndTo
    int map;       // pass 1 XMAP: middle segment whose map it writes (sj - 1), else -1
    bool from_sent;  // pass 2: the entry chain starts from S_1 (segment 1's entry state)
};
constexpr Job carry_job(int nseg, int pass, int kind) {
    if (nseg <= 1) return Job{0, kFromState, true, true, kEndS, -1, false};
    if (pass == 1) {
        if (kind == 0) return Job{0, kFromState, true, true, kEndSent, -1, false};
        const int sj = (kind + 1) / 2;
        if (kind & 1) return Job{sj, kFromZero, false, true, kEndRseg, -1, false};
        return Job{sj, kFromIdentity, false, false, kEndNone, sj - 1, false};
    }
    const int sj = kind + 1;
    return Job{sj, kFromState, true, true, sj == nseg - 1 ? kEndS : kEndNone, -1, true};
}

// The carry launches of one prefill call. Whole-head workgroups are 8 waves of one
// 16-column tile each; half-head workgroups are 4 such waves plus a loader wave. A head
// is split over two workgroups when that still fits one round of the CUs, and for
// packed prompts when it fits two (their chains differ in length and, dispatched
// longest first, the halves finish sooner). The segmented carry runs pass 1 on
// whole-head workgroups (2 nseg - 3 per head) and pass 2 on half-head ones
// (2 (nseg - 1) per head). With `whole` (the gated RMSNorm fused into the output
// store, which needs all 128 columns of a token in one workgroup) every launch uses
// whole-head workgroups: pass 2 then runs nseg - 1 per head.
constexpr int kSortMax = 256;   // packed sequences ranked by length in every carry workgroup
struct CarryLaunch {
    bool half;        // half-head workgroups (4 waves + loader) or whole-head ones (8 waves)
    int pass;         // 0 unsegmented, else 1 or 2
    long long units;  // heads x kinds: workgroups = units * (half ? 2 : 1)
};
struct CarryPlan { int nseg, count; CarryLaunch l[2]; };
constexpr CarryPlan carry_plan(int B, int L, int N, int Hv, bool ragged, int cus, bool whole = false) {
    CarryPlan p{};
    p.nseg = imin(segments(B, L, N, Hv, ragged, kLayoutCUs, whole), segments(B, L, N, Hv, ragged, cus, whole));
    const long long heads = static_cast<long long>(N) * Hv;
    if (heads <= 0) return p;
    if (p.nseg > 1) {
        p.count = 2;
        p.l[0] = CarryLaunch{false, 1, (2 * p.nseg - 3) * heads};
        p.l[1] = CarryLaunch{!whole, 2, (p.nseg - 1) * heads};
    } else {
        const bool split = 2 * heads <= cus || (ragged && N <= kSortMax && heads <= cus);
        p.count = 1;
        p.l[0] = CarryLaunch{split && !whole, 0, heads};
    }
    return p;
}

// ---- carry LDS stage ----------------------------------------------------------------
// A workgroup of NW waves owns CPW = NW * NTW * 16 columns of one head's state. One
// stage holds, for one chunk and head, in 16-byte granules:
//   W [64][16 granules]  Q [64][16]  KT [128][8]  P [64][8]  U^T [CPW][8] (this
//   workgroup's columns, tokens along the row)  coefficients [40]
// Granule j of row r sits at position j ^ (r mod rowgranules) of its row, which
// spreads the 16 rows one MFMA operand read touches over the banks. Every region
// starts on a 1 KB boundary: it is filled by wave-wide 1 KB loads (64 lanes x 16 B).
template <int CPW>
struct Stage {
    static constexpr int W = 0, Q = 1024, KT = 2048, P = 3072, U = 3584;   // granules
    static constexpr int UG = CPW / 8;                 // U^T rows per 8 (the region is 64 x UG granules)
    static constexpr int CF = U + 64 * UG;
    static constexpr int END = CF + COEF / 4;
    static constexpr int INSTR = (END + 63) / 64;      // wave-wide 1 KB loads
    static constexpr int BYTES = INSTR * 1024;
};

// One lane's part of a wave-wide 1 KB load into a stage: source row and granule (the
// element offset in the source is row * rowstride + 8 * gran) and the 1 KB slot of the
// stage it lands in (lane l fills bytes 16 l .. 16 l + 15 of it, i.e. position l % rg of
// row l / rg of the slot's rows, which is granule gran after the swizzle).
struct LaneLoad { int row, gran, slot; };
// rows of 16 granules (W, Q, the state maps): a load covers 4 rows; q = load index
// within the region
constexpr LaneLoad load16(int region_slot0, int q, int lane) {
    const int row = 4 * q + (lane >> 4);
    return LaneLoad{row, (lane & 15) ^ (row & 15), region_slot0 + q};
}
// rows of 8 granules (K^T, P, U^T): a load covers 8 rows
constexpr LaneLoad load8(int region_slot0, int q, int lane) {
    const int row = 8 * q + (lane >> 3);
    return LaneLoad{row, (lane & 7) ^ (row & 7), region_slot0 + q};
}
// The kernels issue a wave's loads of a region as load index q = wave + nw * i,
// i = 0, 1, ...: with nw a multiple of 4 the granule swizzle is the same for every i,
// so load i is load 0 shifted by a constant number of rows and slots (a lane base plus
// a constant stride in the address). The bounds model checks step16 (step8) against
// load16 (load8) for every wave, lane and i.
constexpr LaneLoad step16(LaneLoad l0, int nw, int i) { return LaneLoad{l0.row + 4 * nw * i, l0.gran, l0.slot + nw * i}; }
constexpr LaneLoad step8(LaneLoad l0, int nw, int i) { return LaneLoad{l0.row + 8 * nw * i, l0.gran, l0.slot + nw * i}; }

}  // namespace plan
}  // namespace gdn
