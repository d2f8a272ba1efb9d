// kvq_attn4.h -- pieces of the INT4 decode-attention kernels shared by the VALU kernel
// (kvq_attn_mha4.hip) and the matrix-core kernel (kvq_attn_gqa4.hip): the fused append of the
// decode step's token and the V register layout both kernels use.
//
// V registers: lane l holds the 16 bytes at (l / 16) * 256 + (l % 16) * 16 of its tile -- tokens
// 4 (l / 16) .. +3 of the dims l % 16 + 16 r (r = 0..7), unit r in bits 16 (r % 2) .. +15 of dword
// r / 2 -- in both kernels.
#pragma once

#include "kvq_attn.h"
#include "kvq_int4.h"

namespace kvq {

// The appended token of a fused decode step, encoded with the append kernel's arithmetic: lane l
// holds K dims 2l, 2l + 1 and V dims 2l, 2l + 1 of the new row.  The token's 64 K bytes go to LDS
// in chunk order (byte l = dims 2l, 2l + 1), its 128 V codes to LDS by dim.
struct NewToken4 {
    int slot;
    f32x2 ks, vs;     // (scale, zero point) of the K and V rows
};

__device__ __forceinline__ NewToken4 new_token4(const KernelParams& a, int b, int g, int n, int lane,
                                                uint8_t* lds_k, uint8_t* lds_v) {
#pragma clang fp contract(off)
    NewToken4 nt;
    nt.slot = (n - 1) % kBlock;
    const size_t row = ((size_t)b * a.Hkv + g) * (kDim / 2);
    const uint32_t kw = reinterpret_cast<const uint32_t*>(a.k_new)[row + lane];
    const uint32_t vw = reinterpret_cast<const uint32_t*>(a.v_new)[row + lane];
    const float k0 = half_bits_to_float(kw & 0xFFFFu), k1 = half_bits_to_float(kw >> 16);
    const float v0 = half_bits_to_float(vw & 0xFFFFu), v1 = half_bits_to_float(vw >> 16);
    const float kz = wave_min(fminf(k0, k1)), vz = wave_min(fminf(v0, v1));
    const float ksc = (wave_max(fmaxf(k0, k1)) - kz) / 15.0f;
    const float vsc = (wave_max(fmaxf(v0, v1)) - vz) / 15.0f;
    lds_k[lane] = (uint8_t)(encode_int4(k0, kz, ksc) | (encode_int4(k1, kz, ksc) << 4));
    lds_v[2 * lane] = (uint8_t)encode_int4(v0, vz, vsc);
    lds_v[2 * lane + 1] = (uint8_t)encode_int4(v1, vz, vsc);
    nt.ks = f32x2{ksc, kz};
    nt.vs = f32x2{vsc, vz};
    __builtin_amdgcn_wave_barrier();
    return nt;
}

__device__ __forceinline__ uint32_t set_nibble(uint32_t w, int i, uint32_t q) {
    const int sh = 4 * i;
    return (w & ~(0xFu << sh)) | (q << sh);
}

// The appended token's stores, held back until the wave has read all its tiles (as in the 8-bit
// kernel): its K bytes and this lane's patched 16 V bytes wait in LDS (lds_k, lds_vrow[lane]), so
// that no registers are held for them across the attention loop.
struct PendingAppend4 {
    int blk;       // -1 when nothing is pending (wave-uniform)
    int slot;
    f32x2 ks, vs;
};

// Store a pending token: 16 K bytes in each of the four chunks (lanes 0..3, from LDS), the token's
// quad block of the V tile (its 16 lanes rewrite their 16 bytes with the new nibbles in place; the
// other tokens' nibbles are written back unchanged -- this wave is the tile's only reader and
// writer), and the (scale, zero point) pairs.
__device__ __forceinline__ void flush_append4(const KernelParams& a, PendingAppend4& pa,
                                              const uint8_t* lds_k, const u32x4* lds_vrow, int g, int lane) {
    if (pa.blk < 0) return;
    const size_t tile = ((size_t)pa.blk * a.Hkv + g) * kTileBytes4;
    uint8_t* kt = const_cast<uint8_t*>(a.kc) + tile;
    uint8_t* vt = const_cast<uint8_t*>(a.vc) + tile;
    if (lane < 4)
        __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(lds_k)[lane],
                                    reinterpret_cast<u32x4*>(kt + k_byte4(pa.slot, 32 * lane)));
    if ((lane >> 4) == (pa.slot >> 2))
        __builtin_nontemporal_store(lds_vrow[lane], reinterpret_cast<u32x4*>(vt + v_byte4(pa.slot & ~3, lane & 15)));
    if (lane == 0) {
        const size_t so = ((size_t)pa.blk * a.Hkv + g) * kBlock + pa.slot;
        reinterpret_cast<f32x2*>(const_cast<float*>(a.ks))[so] = pa.ks;
        reinterpret_cast<f32x2*>(const_cast<float*>(a.vs))[so] = pa.vs;
    }
    pa.blk = -1;
}

// Replace token `slot`'s V nibbles in the registers of the 16 lanes of its quad (its nibble in each
// of their eight units), from the token's codes in LDS (by dim).
__device__ __forceinline__ void patch_v_quad(u32x4& v, int slot, const uint8_t* lds_v, int lane) {
    if ((lane >> 4) == (slot >> 2)) {
        const int dlo = lane & 15, i = slot & 3;
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int r = 0; r < 8; ++r)
            w[r / 2] = set_nibble(w[r / 2], 4 * (r % 2) + i, lds_v[dlo + 16 * r]);
        v = u32x4{w[0], w[1], w[2], w[3]};
    }
}

}  // namespace kvq
