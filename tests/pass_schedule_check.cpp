// Host check of the one-launch compress schedule (pass_item and pass_plan
// in sz_internal.h, the functions the kernel calls): for every shape in a
// grid of (tensors, sample items, main items, lag -- up to 5 stages more
// than the tensor count, since a lone large tensor runs with the minimum
// lag of 4), every work item appears exactly once among the item indices (workgroup ids),
// nothing lies past the last one, and
// for each tensor its sample items come before its provisional item, which
// comes before its main items, which come before its final item -- the
// order the kernel's waits rely on (each waits only for lower workgroup ids).
// Prints "ok <shapes checked>".
#include <cstdio>
#include <map>
#include <tuple>

#include "sz_internal.h"

int main() {
    long shapes = 0;
    for (uint32_t T = 1; T <= 9; ++T)
        for (uint32_t S = 1; S <= 4; ++S)
            for (uint32_t M = 1; M <= 5; ++M)
                for (uint32_t lag = 1; lag <= T + 5; ++lag) {
                    sz::CompressArgs a{};
                    a.enc.count = T;
                    a.sample_items = S;
                    a.main_items = M;
                    a.lag = lag;
                    const sz::PassPlan plan = sz::pass_plan(a);
                    const uint64_t total = uint64_t(T) * (S + 1 + M + 1);
                    const uint32_t per[4] = {S, 1, M, 1};
                    std::map<std::tuple<uint32_t, uint32_t, uint32_t>, uint64_t> at;
                    for (uint64_t k = 0; k < total; ++k) {
                        const sz::PassItem it = sz::pass_item(k, plan);
                        if (it.kind >= sz::kItemNone || it.t >= T) return std::printf("bad item at %llu\n", (unsigned long long)k), 1;
                        if (it.idx >= per[it.kind]) return std::printf("index out of range\n"), 1;
                        if (!at.emplace(std::make_tuple(it.kind, it.t, it.idx), k).second) return std::printf("duplicate\n"), 1;
                    }
                    if (at.size() != total) return std::printf("missing items\n"), 1;
                    if (sz::pass_item(total, plan).kind != sz::kItemNone) return std::printf("past the end\n"), 1;
                    for (uint32_t t = 0; t < T; ++t) {
                        const uint64_t prov = at[std::make_tuple(uint32_t(sz::kItemProvisional), t, 0u)];
                        const uint64_t fin = at[std::make_tuple(uint32_t(sz::kItemFinal), t, 0u)];
                        if (prov > fin) return std::printf("final before provisional\n"), 1;
                        for (uint32_t i = 0; i < S; ++i)
                            if (at[std::make_tuple(uint32_t(sz::kItemSample), t, i)] > prov)
                                return std::printf("sample after provisional\n"), 1;
                        for (uint32_t i = 0; i < M; ++i) {
                            const uint64_t m = at[std::make_tuple(uint32_t(sz::kItemMain), t, i)];
                            if (m < prov) return std::printf("main before provisional\n"), 1;
                            if (m > fin) return std::printf("main after final\n"), 1;
                        }
                    }
                    ++shapes;
                }
    std::printf("ok %ld\n", shapes);
    return 0;
}
