"""Print the twiddle table of fft_conv.hip: e^{-2 pi i j / 64} for j < 32,
as cos and sin rounded to the nearest binary32 (from binary64 numpy), so
that every length-n transform (n | 64) takes its factors from it:
e^{-2 pi i j / n} = table[j * 64 / n].  Run once when the table changes:

    python memory_efficient_activation_amd/csrc/gen_fft_twiddles.py
"""

import numpy as np

j = np.arange(32)
ang = 2.0 * np.pi * j / 64.0
c = np.cos(ang).astype(np.float32)
s = np.sin(ang).astype(np.float32)
# Exact values where they are exact.
c[16], s[0], s[16] = 0.0, 0.0, 1.0


def fmt(a):
    return ",\n    ".join(", ".join(f"{float(v):.9e}f" for v in a[i:i + 4]) for i in range(0, 32, 4))


print("constexpr float kCos64[32] = {\n    " + fmt(c) + "};")
print("constexpr float kSin64[32] = {\n    " + fmt(s) + "};")
