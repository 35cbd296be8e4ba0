// Host check of the one-launch compress schedule (pass_item in
// sz_internal.h, the same function the kernel calls): for every shape in a
// grid of (tensors, counting items, encode items, lag), every work item
// appears exactly once among the tickets, and each tensor's counting items
// come before its codebook item, which comes before its encode items -- the
// order the kernel's waits rely on.  Prints "ok <shapes checked>".
#include <cstdio>
#include <map>
#include <tuple>
#include <vector>

#include "sz_internal.h"

int main() {
    using sz::pass_item;
    long shapes = 0;
    for (uint32_t T = 1; T <= 9; ++T)
        for (uint32_t H = 1; H <= 4; ++H)
            for (uint32_t E = 0; E <= 4; ++E)
                for (uint32_t lag = 1; lag <= T; ++lag) {
                    const uint64_t total = uint64_t(T) * (H + 1 + E);
                    std::map<std::tuple<uint32_t, uint32_t, uint32_t>, uint64_t> at;
                    for (uint64_t k = 0; k < total; ++k) {
                        const sz::PassItem it = pass_item(k, T, H, E, lag);
                        if (it.kind == sz::kItemNone || it.t >= T) return std::printf("bad item at %llu\n", (unsigned long long)k), 1;
                        if ((it.kind == sz::kItemCount && it.idx >= H) || (it.kind == sz::kItemEncode && it.idx >= E) ||
                            (it.kind == sz::kItemCodebook && it.idx != 0))
                            return std::printf("index out of range\n"), 1;
                        if (!at.emplace(std::make_tuple(it.kind, it.t, it.idx), k).second) return std::printf("duplicate\n"), 1;
                    }
                    if (at.size() != total) return std::printf("missing items\n"), 1;
                    if (pass_item(total, T, H, E, lag).kind != sz::kItemNone) return std::printf("past the end\n"), 1;
                    for (uint32_t t = 0; t < T; ++t) {
                        const uint64_t cb = at[std::make_tuple(uint32_t(sz::kItemCodebook), t, 0u)];
                        for (uint32_t i = 0; i < H; ++i)
                            if (at[std::make_tuple(uint32_t(sz::kItemCount), t, i)] > cb) return std::printf("count after codebook\n"), 1;
                        for (uint32_t i = 0; i < E; ++i)
                            if (at[std::make_tuple(uint32_t(sz::kItemEncode), t, i)] < cb) return std::printf("encode before codebook\n"), 1;
                    }
                    ++shapes;
                }
    std::printf("ok %ld\n", shapes);
    return 0;
}
