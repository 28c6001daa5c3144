/*
 * FNV-1a content fingerprint of a tensor, for run logs (the weight_fingerprint
 * function of the weight_cache.rs rustdoc source view): the 64-bit FNV-1a
 * hash over every byte, then n_in and n_out each folded in as one 64-bit word
 * the same way.  A compiled copy of synth.fnv1a64_py (the pure-Python
 * statement of the same hash, which pins it) for tensors of tens of MB.
 */
#include <stddef.h>
#include <stdint.h>

uint64_t synth_fnv1a64(const uint8_t* data, size_t n, uint64_t n_in, uint64_t n_out)
{
    const uint64_t prime = 0x100000001B3ull;
    uint64_t h = 0xCBF29CE484222325ull;
    for (size_t i = 0; i < n; ++i) h = (h ^ data[i]) * prime;
    h = (h ^ n_in) * prime;
    h = (h ^ n_out) * prime;
    return h;
}
