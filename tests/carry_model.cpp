// Host-side bounds model of the MFMA prefill's carry kernel (and of the chunk kernel's
// blockIdx map and raw value loads). It includes the index header the kernels themselves compute every
// address from (gdn_prefill_plan.hpp) and, for every launch configuration the launcher
// can choose, replays each workgroup's job: its segment, entry state, every stage load
// (global source row and granule, LDS slot), the state-map prologue of the second pass,
// the outputs and end states it writes; it checks every offset against the size of the
// buffer it indexes and every LDS slot against its stage region, counts the barriers
// each wave role executes, and replays the prologue's hand-encoded vmcnt waits against
// the loads each compute wave has issued. Segment 0's weight is swept over 4..7 eighths
// (the kernels use 5), and every configuration is replayed twice: as planned, and with
// the gated RMSNorm fused (whole-head workgroups only, the second pass included, and
// the gate rows read beside the outputs). Exit status 0 and a summary line when every
// check holds; the first violation is printed and the exit status is 1.
//
// Build and run: g++ -O2 -std=c++17 -I linear_attention_sequence_amd/csrc tests/carry_model.cpp
// An argument plants one mistake the model must report (exit status 1): wait32 (the
// prologue waits for twice the loads of one map), loader_barrier (the loader wave
// executes one barrier more than the compute waves), tail_row (the last chunk's output
// rows run one past the sequence), seg0_wide (segment 0's weight empties later segments).
#include "gdn_prefill_plan.hpp"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <string>
#include <vector>

using namespace gdn::plan;

namespace {

long long g_checks = 0;
std::string g_ctx;
std::string g_plant;   // a planted mistake (argv[1]) that the model must catch

#define REQUIRE(cond)                                                                      \
    do {                                                                                   \
        ++g_checks;                                                                        \
        if (!(cond)) {                                                                     \
            std::fprintf(stderr, "VIOLATION line %d: %s\n  in %s\n", __LINE__, #cond, g_ctx.c_str()); \
            std::exit(1);                                                                  \
        }                                                                                  \
    } while (0)

// the kernels' layout constants that are not in the header (gdn_prefill_mfma.hip)
constexpr int kZeroTile = -(1 << 20);
constexpr int kMapRowStride = D + 8;   // LDS row stride (halfs) of the map planes written by pass 1

struct Config {
    int B, L, N, Hk, Hv;
    bool ragged;
    std::vector<int> starts, lens;   // per sequence (row-relative start for unpacked)
    int cus, seg0;
};

struct WG {   // one carry workgroup's template shape
    int NW, NTW;
    bool LW;
    int NL;       // loader waves (with LW)
    int CPW() const { return NW * NTW * 16; }
};

template <int CPW>
void check_stage_geometry(int NW) {
    using SG = Stage<CPW>;
    // regions start on 1 KB slots and are disjoint, in order, inside the stage
    REQUIRE(SG::W % 64 == 0 && SG::Q % 64 == 0 && SG::KT % 64 == 0 && SG::P % 64 == 0 && SG::U % 64 == 0 &&
            SG::CF % 64 == 0);
    REQUIRE(SG::W + 64 * 16 <= SG::Q && SG::Q + 64 * 16 <= SG::KT && SG::KT + 128 * 8 <= SG::P &&
            SG::P + 64 * 8 <= SG::U && SG::U + CPW * 8 <= SG::CF && SG::CF + COEF / 4 <= SG::END);
    REQUIRE(SG::BYTES >= SG::END * 16 && 2 * SG::BYTES <= 160 * 1024);
    struct R { int slot0, nload, rows, rowgran; bool sixteen; int endslot; };
    const R regions[] = {
        {SG::W / 64, 16 / NW, 64, 16, true, SG::Q / 64},
        {SG::Q / 64, 16 / NW, 64, 16, true, SG::KT / 64},
        {SG::KT / 64, 16 / NW, 128, 8, false, SG::P / 64},
        {SG::P / 64, 8 / NW == 0 ? 1 : 8 / NW, 64, 8, false, SG::U / 64},
        {SG::U / 64, CPW / 8 / NW, CPW, 8, false, SG::CF / 64},
    };
    for (const R& r : regions) {
        // every (row, granule) of the region is loaded exactly once, into its own slot
        std::vector<int> seen(static_cast<size_t>(r.rows) * r.rowgran, 0);
        for (int w = 0; w < NW; ++w)
            for (int i = 0; i < r.nload; ++i) {
                if (w + NW * i >= r.rows * r.rowgran / 64) continue;   // P with NW = 8: one load per wave
                for (int lane = 0; lane < 64; ++lane) {
                    const LaneLoad l = r.sixteen ? load16(r.slot0, w + NW * i, lane) : load8(r.slot0, w + NW * i, lane);
                    const LaneLoad l0 = r.sixteen ? load16(r.slot0, w, lane) : load8(r.slot0, w, lane);
                    const LaneLoad ls = r.sixteen ? step16(l0, NW, i) : step8(l0, NW, i);
                    REQUIRE(ls.row == l.row && ls.gran == l.gran && ls.slot == l.slot);
                    REQUIRE(l.row >= 0 && l.row < r.rows && l.gran >= 0 && l.gran < r.rowgran);
                    REQUIRE(l.slot >= r.slot0 && l.slot < r.endslot && l.slot < SG::INSTR);
                    // the granule lands where the swizzled read of (row, gran) looks for it
                    const int pos_in_slot = lane;   // 16-byte position inside the 1 KB slot
                    const int lds_row = (l.slot - r.slot0) * (64 / r.rowgran) + pos_in_slot / r.rowgran;
                    REQUIRE(lds_row == l.row && (pos_in_slot % r.rowgran) == (l.gran ^ (l.row % r.rowgran)));
                    ++seen[static_cast<size_t>(l.row) * r.rowgran + l.gran];
                }
            }
        for (int v : seen) REQUIRE(v == 1);
    }
}

int sort_rank_sequence(const Config& c, int r) {
    // sequence of rank r: lengths descending, ties by index (as sequence_of_rank)
    std::vector<int> idx(c.N);
    std::iota(idx.begin(), idx.end(), 0);
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return c.lens[a] > c.lens[b]; });
    return idx[r];
}

// The state-map loads of the second pass's prologue: 16 loads of 1 KB per compute wave
// and map, rows of 16 granules over the hi and lo planes (2 D rows). Returns the largest
// element offset past a map's base that any lane reads (+ 8: one granule).
size_t check_map_geometry(int NW, int BYTES) {
    const int MI = 2 * D / 4 / NW;
    size_t top = 0;
    std::vector<int> seen(2 * D * 16, 0);
    for (int w = 0; w < NW; ++w)
        for (int k = 0; k < MI; ++k)
            for (int lane = 0; lane < 64; ++lane) {
                const LaneLoad l = load16(0, w + NW * k, lane);
                const LaneLoad ls = step16(load16(0, w, lane), NW, k);
                REQUIRE(l.row == ls.row && l.gran == ls.gran && l.slot == ls.slot);
                REQUIRE(l.row < 2 * D && l.gran < 16 && (l.slot + 1) * 1024 <= BYTES);
                ++seen[l.row * 16 + l.gran];
                top = std::max(top, static_cast<size_t>(l.row) * D + 8 * l.gran + 8);
            }
    for (int v : seen) REQUIRE(v == 1);   // both planes, every granule, once
    return top;
}

// The first chunk slot of sequence n as the kernels take it: n times the chunks per row
// unpacked; packed, the table the front kernel writes (64-bit prefix sums of the chunk
// counts, clamped to the slot count), whose entries n and n + 1 lie inside its region
// and which, for sequences that fit, equals the plain sum over the sequences before.
std::vector<int> slot_table(const Config& c, const Layout& lay) {
    std::vector<int> t(static_cast<size_t>(c.N) + 1);
    long long run = 0;
    for (int n = 0; n <= c.N; ++n) {
        t[n] = static_cast<int>(std::min(run, static_cast<long long>(lay.nc_max)));
        if (n < c.N) run += chunks_of_len(c.lens[n]);
    }
    return t;
}

int first_slot(const Config& c, const Layout& lay, const std::vector<int>& t, int n) {
    if (!c.ragged) return n * chunks_of_len(c.L);
    REQUIRE(static_cast<size_t>(n) + 1 < lay.n_cbase && lay.cbase + lay.n_cbase * 4 <= lay.bytes);
    long long sum = 0;
    for (int m = 0; m < n; ++m) sum += chunks_of_len(c.lens[m]);
    REQUIRE(sum >= lay.nc_max || t[n] == sum);
    return t[n];
}

// The chunk kernel's lookup of slot id: the sequence and its chunk index (binary search
// of the table for packed prompts), or false for a slot no sequence fills.
bool slot_owner(const Config& c, const std::vector<int>& t, int id, int* n_out, int* c_out) {
    if (!c.ragged) {
        const int per = chunks_of_len(c.L);
        if (per == 0 || id >= c.N * per) return false;
        *n_out = id / per;
        *c_out = id - *n_out * per;
        return true;
    }
    int lo = 0, hi = c.N - 1, n = -1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        REQUIRE(mid >= 0 && mid <= c.N);
        if (t[mid] <= id) { n = mid; lo = mid + 1; } else { hi = mid - 1; }
    }
    if (n < 0 || id >= t[n + 1]) return false;
    *n_out = n;
    *c_out = id - t[n];
    return true;
}

void model_launch(const Config& c, const Layout& lay, int nseg, const CarryLaunch& cl, bool norm) {
    // the launcher's choice: half-head workgroups with one loader wave, two in the second pass
    const WG wg = cl.half ? WG{4, 1, true, cl.pass == 2 ? 2 : 1} : WG{8, 1, false, 1};
    if (wg.LW) {   // loader li issues the stage shares of compute waves li + NL k: each share exactly once
        std::vector<int> share(wg.NW, 0);
        for (int li = 0; li < wg.NL; ++li)
            for (int k = 0; k < wg.NW / wg.NL; ++k) ++share[li + wg.NL * k];
        for (int v : share) REQUIRE(v == 1);
    }
    REQUIRE(!norm || (!wg.LW && wg.NTW == 1 && wg.CPW() == D));   // the fused norm needs whole-head workgroups
    const int CPW = wg.CPW(), NS = 128 / CPW, nh = c.N * c.Hv;
    const int NK = carry_kinds(nseg, cl.pass);
    const long long blocks = cl.units * NS;
    REQUIRE(blocks == static_cast<long long>(NK) * NS * nh);
    const int BYTES = CPW == 64 ? Stage<64>::BYTES : Stage<128>::BYTES;
    const int UG = CPW / 8;
    const size_t map_top = check_map_geometry(wg.NW, BYTES);
    const size_t tiles = static_cast<size_t>(c.N) * c.Hv * D * D;
    const size_t S_elems = tiles, o_elems = static_cast<size_t>(c.B) * c.L * c.Hv * D;
    std::vector<int> covered(static_cast<size_t>(NK) * NS * nh, 0);
    const bool sort = c.ragged && c.N <= kSortMax;
    const std::vector<int> table = c.ragged ? slot_table(c, lay) : std::vector<int>();
    for (long long blk = 0; blk < blocks; ++blk) {
        const CarryUnit un = carry_unit(static_cast<int>(blk), NK * NS, c.N, c.Hk, c.Hv);
        REQUIRE(un.slice >= 0 && un.slice < NK * NS && un.n >= 0 && un.n < c.N && un.h >= 0 && un.h < c.Hv);
        ++covered[static_cast<size_t>(un.slice) * nh + un.n * c.Hv + un.h];
        const int cs = un.slice % NS, kind = un.slice / NS, h = un.h;
        int n = un.n;
        if (sort) n = sort_rank_sequence(c, n);
        const int f = c.Hv / c.Hk, hk = h / f;
        const int base = first_slot(c, lay, table, n);
        int nch = chunks_of_len(c.lens[n]);
        if (base + nch > lay.nc_max) nch = lay.nc_max - base;
        if (nch <= 0) continue;   // the whole workgroup returns before any barrier
        const Job job = carry_job(nseg, cl.pass, kind);
        REQUIRE(job.sj >= 0 && job.sj < (nseg > 1 ? nseg : 1));
        const size_t tile = (static_cast<size_t>(n) * c.Hv + h) * D * D;
        const int ucol0 = cs * CPW;
        REQUIRE(ucol0 + CPW <= D);
        const size_t row_tok = static_cast<size_t>(c.ragged ? 0 : n) * c.L + c.starts[n];
        // entry chains the second pass can take: from S_1 or after a zero map m0 in 1 .. sj-1
        std::vector<int> m0s{0};
        if (job.from_sent)
            for (int i = 1; i <= job.sj - 1; ++i) m0s.push_back(i);
        for (int m0 : m0s) {
            char buf[256];
            std::snprintf(buf, sizeof buf, "B=%d L=%d N=%d Hk=%d Hv=%d ragged=%d cus=%d seg0=%d nseg=%d pass=%d half=%d "
                          "norm=%d block=%lld n=%d h=%d kind=%d m0=%d", c.B, c.L, c.N, c.Hk, c.Hv, c.ragged, c.cus, c.seg0,
                          nseg, cl.pass, cl.half, norm, blk, n, h, kind, m0);
            g_ctx = buf;
            const int np = (nseg > 1 && cl.pass == 2) ? job.sj - 1 - m0 : 0;
            REQUIRE(np >= 0 && np <= kMaxSeg - 2);
            const bool prologue = wg.NTW == 1 && np > 0;
            REQUIRE(!(np > 0) || prologue);   // maps are only ever formed by one-tile waves
            const int cb = nseg > 1 ? seg_begin(nch, nseg, job.sj, c.seg0) : 0;
            const int ce = nseg > 1 ? seg_begin(nch, nseg, job.sj + 1, c.seg0) : nch;
            REQUIRE(cb >= 0 && cb <= ce && ce <= nch);
            // entry state: every (row, column of this workgroup) of S, S_1 or R_m0
            if (job.entry == kFromState) {
                const size_t last = tile + static_cast<size_t>(D - 1) * D + ucol0 + CPW - 1;
                if (m0 > 0) REQUIRE(static_cast<size_t>(m0 - 1) * tiles + last < lay.n_Rseg);
                else if (job.from_sent) REQUIRE(last < lay.n_Sent);
                else REQUIRE(last < S_elems);
            }
            // pass 2: the zero-map scan and the prologue's map, R and exponent reads
            if (job.from_sent) {
                for (int i = job.sj - 1; i >= 1; --i)
                    REQUIRE((static_cast<size_t>(i - 1) * c.N * c.Hv + n * c.Hv + h) * (D / 16) + D / 16 - 1 < lay.n_Mexp);
            }
            if (prologue) {
                const size_t head = static_cast<size_t>(n) * c.Hv + h, nhh = static_cast<size_t>(nh);
                REQUIRE(np * (D / 16) <= wg.NW * 64);   // the exponent loads: one per thread of the compute waves
                for (int t = 0; t < np * (D / 16); ++t)
                    REQUIRE((static_cast<size_t>(m0 + t / (D / 16)) * nhh + head) * (D / 16) + t % (D / 16) < lay.n_Mexp);
                const int MI = 2 * D / 4 / wg.NW;   // 1 KB loads of one map per wave
                REQUIRE(MI * wg.NW * 1024 == 2 * D * D * 2 && MI < 64);   // one map; vmcnt holds it
                for (int i = 1; i <= np; ++i) {
                    const int map = m0 + i - 1;
                    REQUIRE(map >= 0 && map < nseg - 2);
                    const size_t mbase = (static_cast<size_t>(map) * nhh + head) * 2 * D * D;
                    REQUIRE(mbase + map_top <= lay.n_Mhl);
                    // R_map at this lane's accumulator positions: rows 4 g + 16 mt + e, columns col0 + r16
                    const size_t rbase = (static_cast<size_t>(map) * nhh + head) * D * D;
                    REQUIRE(rbase + static_cast<size_t>(D - 1) * D + ucol0 + CPW - 1 < lay.n_Rseg);
                }
                // the vmcnt waits: in-order completion; before map i is read, the wait leaves
                // at most `w` of the wave's latest loads outstanding (w = MI while map i + 1 is
                // in flight, else 0), and the R loads of the previous iteration have been
                // consumed, which completes everything issued before them
                std::vector<int> q;   // issued, possibly outstanding loads: the map index of each (-1: R)
                auto issue = [&](int m, int cnt) { for (int k = 0; k < cnt; ++k) q.push_back(m); };
                issue(1, MI);
                if (np >= 2) issue(2, MI);
                for (int i = 1; i <= np; ++i) {
                    const int wait = (i + 1 <= np) ? (g_plant == "wait32" ? 2 * MI : MI) : 0;
                    const size_t done = q.size() > static_cast<size_t>(wait) ? q.size() - wait : 0;
                    for (size_t k = done; k < q.size(); ++k) REQUIRE(q[k] != i);   // map i has landed
                    q.erase(q.begin(), q.begin() + static_cast<long>(done));
                    issue(-1, 32);                   // R loads, consumed in this iteration
                    q.clear();                       // their use waits for them (and all before)
                    if (i + 2 <= np) issue(i + 2, MI);
                }
            }
            // the !useU stage regions zeroed once: U^T of both stages
            if (!job.useU) REQUIRE((CPW == 64 ? Stage<64>::CF : Stage<128>::CF) * 16 <= BYTES);
            // stage loads, outputs
            const size_t qrows = static_cast<size_t>(c.B) * c.L;
            for (int ch = cb; ch < ce; ++ch) {
                const int id = base + ch;
                REQUIRE(id >= 0 && id < lay.nc_max);
                const int ntc = imin(C, c.lens[n] - ch * C) + (g_plant == "tail_row" ? 1 : 0);
                REQUIRE(ntc >= 1);
                const size_t tok0 = row_tok + static_cast<size_t>(ch) * C;
                REQUIRE(tok0 + ntc <= qrows);
                const size_t wbase = (static_cast<size_t>(id) * c.Hv + h) * C * D;
                const size_t ktbase = (static_cast<size_t>(id) * c.Hk + hk) * D * C;
                const size_t pbase = (static_cast<size_t>(id) * c.Hv + h) * C * C;
                const size_t cfbase = (static_cast<size_t>(id) * c.Hv + h) * COEF;
                // largest row / granule of each region (geometry checked lane by lane)
                REQUIRE(wbase + 63 * D + 8 * 15 + 8 <= lay.n_W);
                if (job.useU) REQUIRE(wbase + static_cast<size_t>(ucol0 + CPW - 1) * C + 8 * 7 + 8 <= lay.n_U);
                REQUIRE(ktbase + 127 * C + 8 * 7 + 8 <= lay.n_KT);
                REQUIRE(cfbase + COEF <= lay.n_coef);
                if (job.outs) {
                    REQUIRE(pbase + 63 * C + 8 * 7 + 8 <= lay.n_P);
                    // q_hat rows past the end load row ntc - 1
                    REQUIRE(((tok0 + ntc - 1) * c.Hk + hk) * D + 8 * 15 + 8 <= lay.n_qh);
                    // output rows tok0 .. tok0 + ntc - 1, columns of this workgroup (and with the
                    // fused norm the gate rows, which have o's shape: rows past the end read row
                    // ntc - 1)
                    REQUIRE(((tok0 + ntc - 1) * c.Hv + h) * D + ucol0 + CPW <= o_elems);
                }
            }
            // end state
            if (job.end == kEndS) REQUIRE(tile + static_cast<size_t>(D - 1) * D + ucol0 + CPW <= S_elems);
            if (job.end == kEndSent) REQUIRE(tile + static_cast<size_t>(D - 1) * D + ucol0 + CPW <= lay.n_Sent);
            if (job.end == kEndRseg)
                REQUIRE(static_cast<size_t>(job.sj - 1) * tiles + tile + static_cast<size_t>(D - 1) * D + ucol0 + CPW <=
                        lay.n_Rseg);
            if (job.map >= 0) {
                REQUIRE(!wg.LW && wg.NTW == 1);   // the map is written by the whole-head pass only
                const size_t m = (static_cast<size_t>(job.map) * tiles + tile) / (D * D);
                REQUIRE(m * (D / 16) + (ucol0 + CPW) / 16 <= lay.n_Mexp);
                REQUIRE(m * 2 * D * D + 2 * D * D <= lay.n_Mhl);
                REQUIRE(2 * D * kMapRowStride * 2 <= 2 * BYTES);   // both planes staged in the two stages
            }
            // barriers per wave role
            const int sortb = sort ? 2 : 0;
            const int compute = sortb + (prologue ? 2 * np : 0) + (ce - cb) + ((!wg.LW && wg.NTW == 1 && job.map >= 0) ? 2 : 0) +
                                (norm && job.outs && ce > cb ? 1 : 0);
            REQUIRE(!(norm && job.outs) || job.map < 0);   // a job forms outputs or writes a map, not both
            if (wg.LW) {
                // every loader wave (one or two) runs the same loop
                const int loader = sortb + (prologue ? 2 * np : 0) + (ce - cb) + (g_plant == "loader_barrier" && np > 1 ? 1 : 0);
                REQUIRE(loader == compute);
            }
            (void)UG;
        }
    }
    for (int v : covered) REQUIRE(v == 1);   // every (slice, slot) has exactly one workgroup
}

// The chunk kernel's raw value loads (v is formed there from the channel-major input):
// for every chunk, token group g8 and both parities of the channel row's offset, the
// two vector loads of the fast path stay inside the channel's row and cover the item's
// conv windows, and the gathered path reads the conv state or positions of the sequence.
void check_value_loads(const Config& c) {
    for (int n = 0; n < c.N; ++n) {
        const int nch = chunks_of_len(c.lens[n]);
        for (int cc = 0; cc < nch; ++cc) {
            const int nt = imin(C, c.lens[n] - cc * C), pc = c.starts[n] + cc * C;
            REQUIRE(nt >= 1 && pc + nt <= c.L);
            const bool vfast = value_fast(cc, nt, pc, c.L);
            for (int g8 = 0; g8 < 8; ++g8) {
                const int p = pc + 8 * g8;
                if (vfast) {
                    for (int ch = 0; ch < 2; ++ch) {               // parities of (ch L + p - 4) over the channels
                        const int parity = (ch * c.L + p - 4) & 1;
                        REQUIRE(parity <= value_load_parity_max(c.L, pc));
                        const int q0 = p - 4 + parity;             // the loads start on a 4-byte boundary
                        REQUIRE(q0 >= 0 && q0 + 12 <= c.L);        // inside the channel's row
                        REQUIRE(q0 <= p - 3 && p + 8 <= q0 + 12);  // the windows of tokens p .. p + 7
                        REQUIRE(p - 3 >= c.starts[n]);             // inside the sequence
                    }
                } else {
                    for (int k = 0; k < 11; ++k) {
                        const int u = cc * C + 8 * g8 - 3 + k;
                        if (u < 0) REQUIRE(u >= -(3));             // conv state slot 3 + u
                        else if (u < c.lens[n]) REQUIRE(c.starts[n] + u < c.L);
                    }
                }
            }
        }
    }
}

void model(const Config& c, bool norm) {
    char buf[160];
    std::snprintf(buf, sizeof buf, "B=%d L=%d N=%d Hk=%d Hv=%d ragged=%d cus=%d seg0=%d", c.B, c.L, c.N, c.Hk, c.Hv,
                  c.ragged, c.cus, c.seg0);
    g_ctx = buf;
    const Layout lay = layout(c.B, c.L, c.N, c.Hk, c.Hv, c.ragged, norm);
    const CarryPlan cp = carry_plan(c.B, c.L, c.N, c.Hv, c.ragged, c.cus, norm);
    REQUIRE(cp.nseg >= 1 && cp.nseg <= lay.nseg + (lay.nseg == 1 ? 0 : 0));
    REQUIRE(cp.nseg == 1 || (cp.nseg >= 3 && cp.nseg <= kMaxSeg && cp.nseg <= lay.nseg));
    // segments are non-empty and ordered for every sequence the launch can meet
    if (cp.nseg > 1)
        for (int n = 0; n < c.N; ++n) {
            const int nch = chunks_of_len(c.lens[n]);
            for (int j = 0; j < cp.nseg; ++j) REQUIRE(seg_begin(nch, cp.nseg, j, c.seg0) < seg_begin(nch, cp.nseg, j + 1, c.seg0));
        }
    // chunk kernel: every (chunk id, V head) exactly once, each id's sequence in range
    {
        std::vector<int> seen(static_cast<size_t>(lay.nc_max) * c.Hv, 0);
        for (int b = 0; b < lay.nc_max * c.Hv; ++b) {
            const ChunkUnit u = chunk_unit(b, lay.nc_max, c.Hk, c.Hv);
            REQUIRE(u.id >= 0 && u.id < lay.nc_max && u.hk >= 0 && u.hk < c.Hk && u.h / (c.Hv / c.Hk) == u.hk);
            ++seen[static_cast<size_t>(u.id) * c.Hv + u.h];
        }
        for (int v : seen) REQUIRE(v == 1);
        // every slot that a sequence fills names that sequence and one of its chunks, and
        // every chunk of every sequence has exactly one slot
        const std::vector<int> t = c.ragged ? slot_table(c, lay) : std::vector<int>();
        std::vector<int> owned(static_cast<size_t>(c.N) * (chunks_of_len(c.L) + 1), 0);
        std::vector<long long> first(static_cast<size_t>(c.N) + 1, 0);
        for (int n = 0; n < c.N; ++n) first[n + 1] = first[n] + chunks_of_len(c.lens[n]);
        for (int id = 0; id < lay.nc_max; ++id) {
            int n = -1, cc = -1;
            if (!slot_owner(c, t, id, &n, &cc)) { REQUIRE(id >= first[c.N]); continue; }
            REQUIRE(n >= 0 && n < c.N && cc >= 0 && cc < chunks_of_len(c.lens[n]) && first[n] + cc == id);
            ++owned[static_cast<size_t>(n) * (chunks_of_len(c.L) + 1) + cc];
        }
        for (int n = 0; n < c.N; ++n)
            for (int cc = 0; cc < chunks_of_len(c.lens[n]); ++cc)
                REQUIRE(owned[static_cast<size_t>(n) * (chunks_of_len(c.L) + 1) + cc] == 1);
    }
    for (int i = 0; i < cp.count; ++i) model_launch(c, lay, cp.nseg, cp.l[i], norm);
    if (!norm) check_value_loads(c);
}

Config unpacked(int B, int L, int Hk, int Hv, int cus, int seg0) {
    Config c{B, L, B, Hk, Hv, false, {}, {}, cus, seg0};
    for (int n = 0; n < B; ++n) { c.starts.push_back(0); c.lens.push_back(L); }
    return c;
}

Config packed(const std::vector<int>& lens, int Hk, int Hv, int cus, int seg0, int tail = 0) {
    Config c{1, 0, static_cast<int>(lens.size()), Hk, Hv, true, {}, lens, cus, seg0};
    int s = 0;
    for (int l : lens) { c.starts.push_back(s); s += l; }
    c.L = s + tail;
    return c;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc > 1) g_plant = argv[1];   // wait32 | loader_barrier | tail_row | seg0_wide
    check_stage_geometry<64>(4);
    check_stage_geometry<128>(8);
    const int heads[][2] = {{16, 32}, {2, 4}, {1, 1}, {4, 4}, {8, 32}, {1, 8}, {2, 2}};
    const int lengths[] = {1, 63, 64, 65, 127, 129, 700, 768, 1000, 1300, 2000, 3000, 4096, 4097, 6000, 8192, 16384};
    const int cus_list[] = {256, 240, 128, 64, 32};
    int configs = 0, segmented = 0;
    const int seg0_hi = g_plant == "seg0_wide" ? 400 : 7;   // a weight that empties later segments
    for (int seg0 = g_plant == "seg0_wide" ? 400 : 4; seg0 <= seg0_hi; ++seg0)
        for (int cus : cus_list)
            for (const auto& hh : heads)
                for (int B = 1; B <= 3; ++B)
                    for (int L : lengths) {
                        const Config c = unpacked(B, L, hh[0], hh[1], cus, seg0);
                        model(c, false);
                        model(c, true);
                        configs += 2;
                        if (carry_plan(B, L, B, hh[1], false, cus).nseg > 1) ++segmented;
                    }
    // packed prompts: the ragged workload's shape, empty and one-token sequences, more
    // sequences than the length ranking handles, a trailing region owned by no sequence
    const std::vector<std::vector<int>> packs = {
        {5106, 3617, 554, 2962, 5386, 4095, 6210, 527}, {100, 3, 64, 0, 65}, {20, 65, 0, 130, 1, 64, 3, 70, 40},
        {1}, {0, 0, 7}, {8192, 8192, 512}, std::vector<int>(300, 17), std::vector<int>(257, 65)};
    for (int seg0 = 4; seg0 <= 7; ++seg0)
        for (int cus : cus_list)
            for (const auto& hh : heads)
                for (const auto& p : packs)
                    for (int tail : {0, 7}) {
                        const Config c = packed(p, hh[0], hh[1], cus, seg0, tail);
                        model(c, false);
                        model(c, true);
                        configs += 2;
                    }
    std::printf("carry model: %d launch configurations (%d segmented), %lld checks, all hold\n", configs, segmented,
                g_checks);
    return 0;
}
