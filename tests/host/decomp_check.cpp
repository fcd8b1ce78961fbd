// Host check of the work split in decomp.h (compiled with g++ by tests/test_decomp.py).
//
// Reads a case from stdin:  B Hkv G window rmax tk P ov  then B lines "L n".
// Walks every workgroup's run exactly as the kernels do and checks that
//   * every real tile of every unit is processed by exactly one workgroup,
//   * a run's part of a unit that holds only set-up positions does nothing,
//   * a unit handled whole by one workgroup is not also split,
//   * the pieces of a split unit are exactly the (workgroup, slot) pairs the
//     combine kernel derives from the unit's own tile range,
//   * no slot of a workgroup is written twice,
//   * no two split units share their first workgroup (the in-kernel merge names a
//     unit's counters by it) and that workgroup exists,
//   * exactly one workgroup of a split unit writes its merge-directory entries (the
//     attention kernel's rule: the run's first segment began inside the unit's real
//     tiles, at most one run length past its first one), and what it derives -- first
//     piece = previous workgroup, last piece, first piece's slot -- is the unit's own.
// Prints "OK <units> <split units> <max pieces>" or "FAIL <reason>".
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <tuple>
#include <vector>

#include "decomp.h"

using namespace dflash;

int main()
{
    Decomp d;
    if (scanf("%d %d %d %d %d %d %d %d", &d.B, &d.Hkv, &d.G, &d.window, &d.rmax, &d.tk, &d.P, &d.ov) != 8)
        return 2;
    std::vector<int> L(d.B), n(d.B);
    for (int r = 0; r < d.B; ++r)
        if (scanf("%d %d", &L[r], &n[r]) != 2)
            return 2;
    int64_t total = 0;
    if (d.ov < 0)
        return 2;
    std::vector<int64_t> rbase(d.B + 1, 0);
    for (int r = 0; r < d.B; ++r) {
        ReqGeom g = req_geom(L[r], n[r], d);
        rbase[r + 1] = rbase[r] + req_work(g, d);
    }
    total = rbase[d.B];
    const int64_t tpw = tiles_per_wg(total, d.P);

    // unit key -> list of (wg, slot, whole)
    std::map<std::tuple<int, int, int>, std::vector<std::tuple<int64_t, int, bool>>> pieces;
    // (request, unit, real tile) -> times processed
    std::map<std::tuple<int, int, int>, int> tile_hits;
    std::set<std::pair<int64_t, int>> slots_used;
    // unit key -> directory entries written: (first piece, last piece, first piece's slot)
    std::map<std::tuple<int, int, int>, std::vector<std::tuple<int64_t, int64_t, int>>> dir_writes;
    for (int64_t wg = 0; wg < d.P; ++wg) {
        const int64_t begin = wg * tpw;
        const int64_t end = std::min<int64_t>(total, begin + tpw);
        if (begin >= end)
            continue;
        int r = 0;
        while (rbase[r + 1] <= begin)
            ++r;
        int64_t rb = rbase[r];
        int64_t pos = begin;
        int seg = 0;
        while (pos < end) {
            ReqGeom g = req_geom(L[r], n[r], d);
            const int64_t w = req_work(g, d);
            if (pos >= rb + w) {
                rb += w;
                ++r;
                continue;
            }
            const Segment sg = run_segment(g, rb, pos, end, d.ov);
            if (sg.next <= pos || sg.t1 > g.ntiles || sg.t0 < 0) {
                printf("FAIL segment bounds\n");
                return 1;
            }
            pos = sg.next;
            if (sg.t0 >= sg.t1)
                continue;
            const bool whole = sg.t0 == 0 && sg.t1 == g.ntiles;
            const int slot = seg == 0 ? 0 : 1;
            for (int t = sg.t0; t < sg.t1; ++t)
                tile_hits[{r, sg.unit, t}]++;
            const int kvh = sg.unit / g.ngroups, grp = sg.unit % g.ngroups;
            pieces[{r, kvh, grp}].push_back({wg, slot, whole});
            if (!whole) {
                if (!slots_used.insert({wg, slot}).second) {
                    printf("FAIL slot written twice wg=%lld slot=%d\n", (long long)wg, slot);
                    return 1;
                }
                // a partial piece must be the first or the last segment of the run
                if (!(seg == 0 || sg.next == end)) {
                    printf("FAIL partial segment in the middle of a run\n");
                    return 1;
                }
                if (slot == 0 && sg.t0 > 0 && sg.t0 <= tpw) {  // the directory's writer
                    const int64_t us = rb + (int64_t)sg.unit * g.uwork;
                    const int64_t kf = wg - 1;
                    const int64_t kl = (us + g.uwork - 1) / tpw;
                    dir_writes[{r, kvh, grp}].push_back({kf, kl, kf * tpw < us ? 1 : 0});
                }
            }
            ++seg;
        }
    }
    for (int r = 0; r < d.B; ++r) {
        ReqGeom g = req_geom(L[r], n[r], d);
        for (int u = 0; u < (g.ngroups ? d.Hkv * g.ngroups : 0); ++u)
            for (int t = 0; t < g.ntiles; ++t) {
                auto it = tile_hits.find({r, u, t});
                const int hits = it == tile_hits.end() ? 0 : it->second;
                if (hits != 1) {
                    printf("FAIL request %d unit %d tile %d hit %d times\n", r, u, t, hits);
                    return 1;
                }
            }
    }
    int split = 0;
    size_t max_pieces = 0;
    std::set<int64_t> first_wgs;
    for (int r = 0; r < d.B; ++r) {
        ReqGeom g = req_geom(L[r], n[r], d);
        for (int kvh = 0; kvh < (g.ngroups ? d.Hkv : 0); ++kvh)
            for (int grp = 0; grp < g.ngroups; ++grp) {
                auto& pl = pieces[{r, kvh, grp}];
                const int unit = kvh * g.ngroups + grp;
                const int64_t us = rbase[r] + (int64_t)unit * g.uwork;
                int64_t kf, kl;
                unit_pieces(g, us, d.ov, tpw, kf, kl);
                const auto& dw = dir_writes[{r, kvh, grp}];
                if (kf == kl) {
                    if (pl.size() != 1 || !std::get<2>(pl[0])) {
                        printf("FAIL unit not whole in one workgroup\n");
                        return 1;
                    }
                    if (!dw.empty()) {
                        printf("FAIL directory entries written for a whole unit\n");
                        return 1;
                    }
                    continue;
                }
                if (dw.size() != 1 || std::get<0>(dw[0]) != kf || std::get<1>(dw[0]) != kl ||
                    std::get<2>(dw[0]) != piece_slot(kf, us, tpw)) {
                    printf("FAIL directory writer of a split unit (%zu writers)\n", dw.size());
                    return 1;
                }
                ++split;
                max_pieces = std::max(max_pieces, pl.size());
                if (kf < 0 || kf >= d.P || !first_wgs.insert(kf).second) {
                    printf("FAIL split units share their first workgroup %lld\n", (long long)kf);
                    return 1;
                }
                if ((int64_t)pl.size() != kl - kf + 1) {
                    printf("FAIL split unit piece count\n");
                    return 1;
                }
                for (int64_t k = kf; k <= kl; ++k) {
                    const int slot = piece_slot(k, us, tpw);  // the combine's rule
                    bool found = false;
                    for (auto& p : pl)
                        if (std::get<0>(p) == k && std::get<1>(p) == slot && !std::get<2>(p))
                            found = true;
                    if (!found) {
                        printf("FAIL combine cannot find piece wg=%lld slot=%d\n", (long long)k, slot);
                        return 1;
                    }
                }
            }
    }
    printf("OK %zu %d %zu\n", pieces.size(), split, max_pieces);
    return 0;
}
