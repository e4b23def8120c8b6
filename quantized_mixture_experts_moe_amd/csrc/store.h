// Expert store on local storage (internal interface used by the pool).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe.h"
#include "moe_internal.h"

namespace moe {

constexpr size_t kStoreAlign = 4096;  // direct I/O: offsets, lengths and buffers
constexpr int kStoreMaxThreads = 64;

size_t store_stride(int D, int F);
// Reads the blobs (layer, experts[i]) into dst[i] (each at least the stride,
// 4096-byte aligned for direct I/O), in pieces of `chunk` bytes spread over
// the store's reader threads; blocks until every piece is read.
moe_status store_read(moe_store *st, int layer, const int32_t *experts, int n, void *const *dst,
                      size_t chunk);
size_t store_blob_bytes(const moe_store *st);
size_t store_stride_of(const moe_store *st);
int store_layers(const moe_store *st);
int store_E(const moe_store *st);
int store_D(const moe_store *st);
int store_F(const moe_store *st);
bool store_direct(const moe_store *st);

}  // namespace moe
