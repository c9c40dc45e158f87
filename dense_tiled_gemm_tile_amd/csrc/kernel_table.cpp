// The kernel instance table: the instances of every kernel translation unit,
// indexed by kernel id.
#include <stdlib.h>

#include "kernel_table.h"

namespace {

struct Table {
    static constexpr int kMax = 128;
    TgKernelDesc k[kMax];
    int n = 0;
    Table() {
        const struct {
            const TgKernelDesc* e;
            int count;
        } parts[] = {{tg_entries_wide16, tg_entries_wide16_count}, {tg_entries_wide32, tg_entries_wide32_count},
                     {tg_entries_wide8, tg_entries_wide8_count},   {tg_entries_stream, tg_entries_stream_count},
                     {tg_entries_rs, tg_entries_rs_count},         {tg_entries_kslice, tg_entries_kslice_count},
                     {tg_entries_wide4, tg_entries_wide4_count},   {tg_entries_wide6, tg_entries_wide6_count},
                     {tg_entries_wide_m16, tg_entries_wide_m16_count}};
        bool seen[kMax] = {};
        for (const auto& part : parts)
            for (int i = 0; i < part.count; ++i) {
                const TgKernelDesc& d = part.e[i];
                // ids are dense, unique and below kMax by construction of the lists
                if (d.id < 0 || d.id >= kMax || seen[d.id]) abort();
                seen[d.id] = true;
                k[d.id] = d;
                if (d.id + 1 > n) n = d.id + 1;
            }
        for (int i = 0; i < n; ++i)
            if (!seen[i]) abort();
    }
};

const Table& table() {
    static const Table t;
    return t;
}

}  // namespace

int tg_kernel_count() { return table().n; }

const TgKernelDesc& tg_kernel(int id) { return table().k[id]; }
